// Dense 1 x 1 layer with a residual, the adapter's wide projections:
//   Y[k][o] = sum_i A[k][i] B[i][o] + bias[o] + R[k][o]
// with B = Wu (the up-projection's forward, Y = X + H2 Wu + bu) or B = Wd^T
// (the down-projection's input gradient, dX = dY + dH1 Wd^T).
// ("SV-TAD: Native Sparse Convolutions for Efficient Temporal Action
// Detection", Overall Architecture and Key Design 3: the bottleneck adapter
// projects the features down to r channels, convolves them and projects them
// back, adding the result to its input.)
//
// At C = 1024 output channels and r = 256 contracted ones a token costs 512
// FLOP per output byte written, and A, R and Y move 4.5 KB per token: the
// layer is bound by HBM, not by the matrix cores.  The kernel is built to
// keep HBM busy:
//   - a workgroup owns one 256-wide block of output channels for its whole
//     life and holds that block of B (K x 256 bf16, 128 KB at K = 256) in LDS
//     in MFMA fragment order, loaded once;
//   - it walks 64-token tiles (tile p, p + P, p + 2P, ... for workgroup p of
//     its channel block), so that all workgroups stream through the tokens
//     together, and the channel blocks of one tile sit on one XCD and share
//     its A rows in L2;
//   - the product is computed transposed, D = B^T A^T (rows = channels,
//     columns = tokens): the token operand of the MFMA is then 8 consecutive
//     A elements of one row, loaded straight from memory (16 bytes per lane,
//     no LDS);
//   - the residual and the output move as whole rows through an LDS tile
//     buffer (below);
//   - each k-step's A registers are refilled with the next tile's A as soon
//     as its MFMAs are issued.
// Measured at C = 1024, r = 256 (58,822 tokens), per launch: 63 us; the
// earlier launch through the gather kernel took 97 us.  Slower variants:
// R and Y moved directly in the MFMA result layout, 8 bytes per lane
// (94 us); the next tile's R requested a tile earlier into registers (the
// compiler then waited for every load at the loop head); 32-token tiles with
// two LDS tile buffers (77 us); 128-wide blocks with two workgroups per
// compute unit (80 us: every A row is then fetched by twice as many waves);
// half of the B block in registers to make room for two 64-token tile
// buffers (512 registers, and the compiler's waits at the head of the
// two-tile loop took every load in flight).
#include "internal.h"
#include "mfma.h"

namespace svc {

constexpr int DR_TOK = 64;        // tokens per tile
constexpr int DR_CB = 256;        // output channels per workgroup
constexpr int DR_THREADS = 256;   // 4 waves, one per SIMD

// B in fragment order: [Co / 256][K / 16][8 channel blocks][64 lanes][8 bf16].
// Piece (ks, j) of channel block cb is the MFMA A-operand fragment of output
// channels cb * 256 + 32 j .. +31 at k-step ks: lane l holds channel
// 32 j + (l & 31) and k = 16 ks + 8 (l >> 5) .. +7.
// trans = 0: B[i][o] = W[i * Co + o] (W is [K][Co], the up-projection's Wu);
// trans = 1: B[i][o] = W[o * K + i] (W is [Co][K], the down-projection's Wd).
__global__ __launch_bounds__(256) void k_repack_dense(const uint16_t* __restrict__ W, uint16_t* __restrict__ Bf,
                                                      int K, int Co, int trans) {
    const int64_t chunks = static_cast<int64_t>(K) * Co / 8;
    for (int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; c < chunks;
         c += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int lane = static_cast<int>(c & 63);
        const int64_t piece = c >> 6;               // (cb * K/16 + ks) * 8 + j
        const int j = static_cast<int>(piece & (DR_CB / 32 - 1));
        const int64_t rest = piece / (DR_CB / 32);
        const int ks = static_cast<int>(rest % (K / 16));
        const int cb = static_cast<int>(rest / (K / 16));
        const int o = cb * DR_CB + 32 * j + (lane & 31);
        const int i0 = 16 * ks + 8 * (lane >> 5);
        uint16_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            v[e] = trans ? W[static_cast<int64_t>(o) * K + i0 + e] : W[static_cast<int64_t>(i0 + e) * Co + o];
        uint4 q;
        q.x = v[0] | (static_cast<uint32_t>(v[1]) << 16);
        q.y = v[2] | (static_cast<uint32_t>(v[3]) << 16);
        q.z = v[4] | (static_cast<uint32_t>(v[5]) << 16);
        q.w = v[6] | (static_cast<uint32_t>(v[7]) << 16);
        reinterpret_cast<uint4*>(Bf)[c] = q;
    }
}

// s_barrier after the LDS accesses only (lgkmcnt(0)); vector memory
// operations stay in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);    // lgkmcnt(0), vmcnt and expcnt unconstrained
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Wave w computes tokens 32 (w & 1) .. +31 of a 64-token tile x output
// channels 128 (w >> 1) .. +127 of the block (4 blocks of 32 x 32, rows =
// channels).  KS = K / 16 k-steps.  R is required; bias may be null.
//
// The residual and the output pass through LDS, so that memory sees whole
// 512-byte rows (16 bytes per lane, 32 lanes per row) rather than the 8-byte
// pieces of the MFMA result layout: the tile's R rows come in by direct
// loads, each lane adds its results to them in place and rounds, and the
// rows go out from LDS; then the next tile's R rows are requested into the
// same buffer, and arrive during that tile's MFMAs.  Row r of the tile
// buffer holds 16-byte chunk c of its row at position c ^ (r mod 32), so
// that the result-layout accesses (32 rows at one chunk) spread over the
// banks.
template <int KS>
__global__ __launch_bounds__(DR_THREADS) void k_dense_res(const uint16_t* __restrict__ A,
                                                          const uint16_t* __restrict__ Bf,
                                                          const uint16_t* __restrict__ bias,
                                                          const uint16_t* __restrict__ R,
                                                          uint16_t* __restrict__ Y, int n, int Co, int per_cb) {
    constexpr int K = 16 * KS;
    constexpr int ROWB = DR_CB * 2;                  // bytes of a tile row (256 channels)
    constexpr int CPR = ROWB / 16;                   // 16-byte chunks per row (32)
    constexpr int RQ = DR_TOK * CPR / DR_THREADS;    // row pieces per thread (8)
    constexpr int NJ = DR_CB / 32;                   // 32-channel blocks of the block (8)
    __shared__ __align__(16) char sB[K * DR_CB * 2];
    __shared__ __align__(16) char sT[DR_TOK * ROWB];

    const int cbs = Co / DR_CB;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int cb = logical % cbs, p = logical / cbs;
    const int tiles = (n + DR_TOK - 1) / DR_TOK;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int th = wave & 1, chh = wave >> 1;
    const int l32 = lane & 31, lhi = lane >> 5;

    typedef __attribute__((address_space(3))) void lds_void_t;
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const rsrc_t rA = make_rsrc(A, static_cast<uint32_t>(n) * K * 2);
    const rsrc_t rR = make_rsrc(R, static_cast<uint32_t>(n) * Co * 2);
    const rsrc_t rY = make_rsrc(Y, static_cast<uint32_t>(n) * Co * 2);
    const uint32_t rowG = static_cast<uint32_t>(Co) * 2, colG = static_cast<uint32_t>(cb) * ROWB;
    // R rows of tile tt into sT: instruction j (by wave j mod 4) fills rows
    // 2j, 2j + 1; lane l takes position l & 31 of row 2j + (l >> 5)
    auto load_rt = [&](int tt) __attribute__((always_inline)) {
#pragma unroll
        for (int jj = 0; jj < DR_TOK / 2 / 4; ++jj) {
            const int j = wave + 4 * jj, row = 2 * j + lhi;
            const uint32_t c = static_cast<uint32_t>(l32 ^ (row & 31));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rR, (lds_void_t*)(sT + j * 1024), 16,
                static_cast<uint32_t>(tt * DR_TOK + row) * rowG + colG + c * 16, 0, 0, 0);
        }
    };

    // this block of B into LDS (direct loads, 1 KB per wave instruction)
    {
        const rsrc_t rB = make_rsrc(Bf + static_cast<int64_t>(cb) * K * DR_CB, static_cast<uint32_t>(K) * DR_CB * 2);
        constexpr int pieces = KS * NJ;
        for (int q = wave; q < pieces; q += DR_THREADS / 64)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void_t*)(sB + q * 1024), 16,
                                                     static_cast<uint32_t>(q * 1024 + lane * 16), 0, 0, 0);
    }
    // bias of this lane's result channels (4 per (jb, g)), bf16 pairs
    u32x2 bv[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int ch = cb * DR_CB + 128 * chh + 32 * (q >> 2) + 8 * (q & 3) + 4 * lhi;
        bv[q] = bias ? *reinterpret_cast<const u32x2*>(bias + ch) : u32x2{0u, 0u};
    }

    // token operand: row (tile token) 32 th + l32, k = 16 ks + 8 lhi .. +7
    const uint32_t aLane = static_cast<uint32_t>(32 * th + l32) * K * 2 + lhi * 16;
    const uint32_t aTile = static_cast<uint32_t>(DR_TOK) * K * 2;
    // Offsets past the end read zeros and drop stores (buffer range checks);
    // a tile index past the last tile is clamped to one past it.
    auto tile_of = [&](int i) { return min(p + i * per_cb, tiles); };
    int t = tile_of(0);
    bf16x8_t a[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const uint4 v = load16(rA, static_cast<uint32_t>(t) * aTile + aLane + ks * 32);
        a[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
    load_rt(t);
    __syncthreads();                       // B block and the first R rows in LDS

    // this lane's result (jb, g) = (q >> 2, q & 3): row 32 th + l32, chunk
    // 16 chh + 4 jb + g, half lhi
    const int trow = 32 * th + l32;
    auto tpos = [&](int q) { return trow * ROWB + (((16 * chh + q) ^ (trow & 31)) * 16) + 8 * lhi; };
    const int pc = tid & (CPR - 1), pr = tid / CPR;   // row pieces: chunk pc of rows pr + 8 q

    for (int i = 0; t < tiles; ++i) {
        // keeps the B fragment reads inside the loop: hoisted out of it (they
        // do not change) they would hold the whole block in registers
        asm volatile("" ::: "memory");
        const int tn = tile_of(i + 1);
        floatx16_t acc[4];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) acc[jb] = zero16();
        // B fragments of k-step ks + 1 are read during k-step ks's MFMAs
        auto bfrags = [&](int ks, bf16x8_t* b) __attribute__((always_inline)) {
#pragma unroll
            for (int jb = 0; jb < 4; ++jb)
                b[jb] = frag_row(reinterpret_cast<const uint16_t*>(sB + ((ks * NJ + 4 * chh + jb) * 64 + lane) * 16));
        };
        bf16x8_t b[4], bn[4];
        bfrags(0, b);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 1 < KS) bfrags(ks + 1, bn);
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) acc[jb] = mfma32(b[jb], a[ks], acc[jb]);
            const uint4 v = load16(rA, static_cast<uint32_t>(tn) * aTile + aLane + ks * 32);
            a[ks] = __builtin_bit_cast(bf16x8_t, v);
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) b[jb] = bn[jb];
        }
        // tile i's R rows in sT for this wave (older than the KS A loads just
        // issued), then for every wave
        __builtin_amdgcn_s_waitcnt(((KS & 15) | ((KS >> 4) << 14)) | (0x7 << 4) | (0xf << 8));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        // (acc + bias) + residual, rounded once to bf16, in place (all reads
        // first: interleaved, each write would wait for the read before it)
        u32x2 rvs[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) rvs[q] = *reinterpret_cast<const u32x2*>(sT + tpos(q));
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const u32x2 rv = rvs[q];
            const floatx16_t& ac = acc[q >> 2];
            const int g = q & 3;
            const float y0 = (ac[4 * g + 0] + __uint_as_float(bv[q].x << 16)) + __uint_as_float(rv.x << 16);
            const float y1 = (ac[4 * g + 1] + __uint_as_float(bv[q].x & 0xffff0000u)) + __uint_as_float(rv.x & 0xffff0000u);
            const float y2 = (ac[4 * g + 2] + __uint_as_float(bv[q].y << 16)) + __uint_as_float(rv.y << 16);
            const float y3 = (ac[4 * g + 3] + __uint_as_float(bv[q].y & 0xffff0000u)) + __uint_as_float(rv.y & 0xffff0000u);
            u32x2 o;
            o.x = f32_to_bf16(y0) | (static_cast<uint32_t>(f32_to_bf16(y1)) << 16);
            o.y = f32_to_bf16(y2) | (static_cast<uint32_t>(f32_to_bf16(y3)) << 16);
            *reinterpret_cast<u32x2*>(sT + tpos(q)) = o;
        }
        // Barriers that wait for LDS only: __syncthreads would also wait for
        // the next tile's loads and this tile's stores.
        lds_barrier();
        // the tile's rows out (chunk pc of rows pr + 8 q)
        u32x4 yv[RQ];
#pragma unroll
        for (int q = 0; q < RQ; ++q) {
            const int row = pr + 8 * q;
            yv[q] = *reinterpret_cast<const u32x4*>(sT + row * ROWB + ((pc ^ (row & 31)) * 16));
        }
#pragma unroll
        for (int q = 0; q < RQ; ++q)
            __builtin_amdgcn_raw_buffer_store_b128(
                yv[q], rY, static_cast<uint32_t>(t * DR_TOK + pr + 8 * q) * rowG + colG + pc * 16, 0, 0);
        lds_barrier();                     // sT read by every wave
        load_rt(tn);
        t = tn;
    }
}

bool dense_res_supported(bool bf16, int K, int Co, int64_t n) {
    return bf16 && (K == 64 || K == 128 || K == 256) && Co > 0 && Co % DR_CB == 0 &&
           n * K * 2 + static_cast<int64_t>(DR_TOK) * K * 2 <= kMaxRange &&
           n * Co * 2 + static_cast<int64_t>(DR_TOK) * Co * 2 <= kMaxRange;
}

size_t dense_res_ws_bytes(int K, int Co) { return static_cast<size_t>(K) * Co * 2; }

hipError_t launch_repack_dense(const uint16_t* W, uint16_t* Bf, int K, int Co, bool trans, hipStream_t stream) {
    const int64_t chunks = static_cast<int64_t>(K) * Co / 8;
    const int blocks = static_cast<int>(std::min<int64_t>((chunks + 255) / 256, 1024));
    hipLaunchKernelGGL(k_repack_dense, dim3(blocks), dim3(256), 0, stream, W, Bf, K, Co, trans ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_dense_res(const uint16_t* A, const uint16_t* Bf, const uint16_t* bias, const uint16_t* R,
                            uint16_t* Y, int64_t n, int K, int Co, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const int cbs = Co / DR_CB;
    const int64_t tiles = (n + DR_TOK - 1) / DR_TOK;
    // one workgroup per compute unit (160 KB of LDS each), split evenly over
    // the channel blocks, never more per block than there are tiles
    const int per_cb = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(tiles, 256 / std::max(1, cbs))));
    const dim3 grid(per_cb * cbs), block(DR_THREADS);
    const int ni = static_cast<int>(n);
    switch (K) {
    case 64: hipLaunchKernelGGL(k_dense_res<4>, grid, block, 0, stream, A, Bf, bias, R, Y, ni, Co, per_cb); break;
    case 128: hipLaunchKernelGGL(k_dense_res<8>, grid, block, 0, stream, A, Bf, bias, R, Y, ni, Co, per_cb); break;
    case 256: hipLaunchKernelGGL(k_dense_res<16>, grid, block, 0, stream, A, Bf, bias, R, Y, ni, Co, per_cb); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace svc
