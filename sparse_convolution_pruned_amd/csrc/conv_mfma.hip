// bf16 gather-GEMM on the CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16,
// fp32 accumulation) for the forward pass and the input gradient.
// ("SV-TAD: Native Sparse Convolutions for Efficient Temporal Action
// Detection", Key Design 2: y_k = sum_j W_j x[N[k, j]] as an implicit GEMM
// with M = tokens, K = 9 * C, N = output channels; -1 entries are zero
// padding.)
//
// One kernel serves both passes and every K x K neighbourhood it is built
// for (TAPS = K * K = 1, 9, 25 or 49; P = TAPS - 1).  It computes
//     out[k][c] = sum_j sum_i A[N[k, j]][i] * B[P - j][c][i]  (+ bias[c]) (+ R[k][c])
// with B stored [tap][output channel][contracted channel]:
//   input gradient: A = dY, B = Wt itself ([TAPS][C_in][C_out]: tap P-j of
//     the weights meets the row gathered through tap j, the mirror of the
//     K x K offsets);
//   forward: A = X, B = V with V[P-j][o][i] = Wt[j][i][o], written by a small
//     repacking kernel into the caller's workspace.
// Every MFMA fragment is then one 16-byte LDS read and every staging copy a
// plain 16-byte copy.
//
// Workgroup: 256 threads = 4 waves (2 x 2); output tile 128 tokens x 128
// channels; each wave 64 x 64 = 2 x 2 blocks of 32 x 32.  Two workgroups fit
// on a compute unit at 3 x 3 (67 KiB of LDS each) and 5 x 5 (78 KiB); one at
// 7 x 7 (96 KiB).  Plain 3 x 3 calls whose 128-token tiles would need one
// more dispatch round than 192-token tiles use the latter: each wave 96 x 64
// = 3 x 2 blocks, a 256-row window, 80 KiB of LDS, still two per compute
// unit.  The 1-D grid is remapped so that
// each XCD runs a contiguous range of tiles (neighbouring token ranges and
// the channel tiles of one range share rows in that XCD's L2).
//
// Neighbour window.  Tokens are packed frame-major and, inside a frame, in
// ascending flat order, so every neighbour of token k lies within
// (K/2)(W+1) packed positions of k and a tile's gathered rows sit in one
// short range [lo, hi].
// The kernel reads the tile's N slice, finds lo/hi, and when the range holds
// at most 192 rows (256 for a 192-token tile) it stages exactly those rows
// (64 channels at a time, 16-byte coalesced loads) in LDS once for all taps;
// A fragments are then read from LDS by row index (N - lo; -1 maps to an
// all-zero row).  Tiles whose rows are spread wider (another packing order,
// grids wider than 31 at 3 x 3) fall back to staging the tile's gathered rows
// tap by tap.  Both modes feed the same MFMA
// sequence, so the result does not depend on the mode.
//
// Pipeline.  The K loop runs over rounds (64-channel chunk, tap).  At the
// start of round r the weight tile of round r + 1 goes from registers into
// the free LDS buffer and the loads of round r + 2 are issued, all ahead of
// round r's MFMAs; the next chunk's window rows load into registers half-way
// through the current chunk.  One barrier per round; each round's 4 k-steps
// are unrolled with all fragment reads issued before the 16 (or 24) MFMAs.  The
// output tile leaves through LDS so that global stores are whole 16-byte row
// pieces.
#include "internal.h"
#include "mfma.h"

namespace svc {

constexpr int CM_BM = 128;              // tokens per tile (two 32-row blocks per wave)
constexpr int CM_BM3 = 192;             // tokens per tile with three 32-row blocks per wave
constexpr int CM_BN = 128;              // output channels per tile
constexpr int CM_KC = 64;               // channels per round
constexpr int CM_WIN = 192;             // window rows held in LDS (more than one tap)
constexpr int CM_LDA = CM_KC + 8;       // 144 B pitch: conflict-free 16-byte row reads
constexpr int CM_LDB = CM_KC;           // weight tile rows: 128 B, XOR-swizzled 16-byte chunks
constexpr int CM_SB = CM_BN * CM_LDB;

// One round: 4 k-steps of 16, all fragments read first, then 8 * MB MFMAs
// (MB 32-row blocks of tokens per wave).
template <int MB>
__device__ __forceinline__ void mma_round(const uint16_t* __restrict__ sA, const uint16_t* __restrict__ sb,
                                          const int arow[MB], floatx16_t acc[MB][2]) {
    constexpr int KS = CM_KC / 16;
    const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 1;
    const int l32 = lane & 31, lhi = lane >> 5;
    bf16x8_t a[KS][MB], b[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int kof = ks * 16 + lhi * 8;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) a[ks][mb] = frag_row(&sA[arow[mb] * CM_LDA + kof]);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
            b[ks][nb] = frag_row(&sb[(wn * 64 + nb * 32 + l32) * CM_LDB + (((2 * ks + lhi) ^ ((l32 >> 1) & 7)) << 3)]);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32(a[ks][mb], b[ks][nb], acc[mb][nb]);
}

// A [n][K], B [TAPS][NO][K], bias [NO] (nullable), res [n][NO] (nullable: a
// residual added before the one rounding to bf16), out [n][NO]; K % 32 == 0,
// NO % 16 == 0.  With PAIR the grid also covers a second problem on the
// same N (`second`: its own A, B, output and channel counts, no bias or
// residual): logical tiles from second.tiles_first on belong to it.  The
// chunk driver pairs a chunk's forward and input gradient this way, so that
// the two small launches fill the chip together.
struct ConvSecond {
    const uint16_t* A;
    const uint16_t* B;
    uint16_t* out;
    int K, NO, tiles_first;
};

// MB = 2: 128-token tiles (every variant).  MB = 3: 192-token tiles, 3 x 3
// neighbourhoods without residual or pair only (80 KiB of LDS, two per
// compute unit); chosen when it needs fewer dispatch rounds (see
// conv_tile_blocks).
template <int TAPS, bool RES, bool PAIR, int MB>
__global__ __launch_bounds__(256, TAPS <= 25 ? 2 : 1) void k_conv_mfma(const uint16_t* __restrict__ A0,
                                                      const int32_t* __restrict__ Nt,
                                                      const uint16_t* __restrict__ B0,
                                                      const uint16_t* __restrict__ bias0,
                                                      const uint16_t* __restrict__ res,
                                                      uint16_t* __restrict__ out0, int n, int K0, int NO0,
                                                      ConvSecond second) {
    // Window rows held in LDS: 192 for a 128-token tile, 256 for a 192-token
    // one (a tile's rows and the neighbours around them).  With one tap the window is the tile's own 128 rows, and two
    // windows are held, double-buffered like the weight tiles: one barrier
    // per round instead of two, and the next window's store no longer waits
    // for every wave to leave the current one.
    static_assert(MB == 2 || (MB == 3 && TAPS == 9 && !RES && !PAIR), "192-token tiles: 3 x 3 plain calls only");
    constexpr int BM = 64 * MB;                    // tokens per tile
    constexpr bool DBW = TAPS == 1;
    constexpr int WIN = DBW ? BM : (MB == 2 ? CM_WIN : 256);
    constexpr int ZROW = WIN;                      // an all-zero row: target of -1 entries
    constexpr int WBUF = (WIN + 1) * CM_LDA;       // one window buffer
    constexpr int WREGS = (WIN * (CM_KC / 8) + 255) / 256;
    __shared__ __align__(16) uint16_t sA[(DBW ? 2 : 1) * WBUF];
    __shared__ __align__(16) uint16_t sB[2][CM_SB];   // weight tiles, written by direct loads
    __shared__ int sN[BM * TAPS];
    __shared__ short sRow[BM * TAPS];
    __shared__ int sLo, sHi;

    // The wave index is uniform; through the scalar unit it keeps every
    // per-wave quantity scalar.
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, lhi = lane >> 5;
    // 1-D grid: logical tile = (token tile, output-channel tile), the
    // output-channel tiles of one token range adjacent and on one XCD.
    int logical = xcd_remap(blockIdx.x, gridDim.x);
    const bool two = PAIR && logical >= second.tiles_first;
    const uint16_t* __restrict__ A = two ? second.A : A0;
    const uint16_t* __restrict__ B = two ? second.B : B0;
    const uint16_t* __restrict__ bias = two ? nullptr : bias0;
    uint16_t* __restrict__ out = two ? second.out : out0;
    const int K = two ? second.K : K0;
    const int NO = two ? second.NO : NO0;
    if (two) logical -= second.tiles_first;
    const int tilesN = (NO + CM_BN - 1) / CM_BN;
    const int64_t k0 = static_cast<int64_t>(logical / tilesN) * BM;
    const int n0 = (logical % tilesN) * CM_BN;
    const int nchunks = (K + CM_KC - 1) / CM_KC;
    const int R = nchunks * TAPS;

    if (tid == 0) { sLo = 0x7fffffff; sHi = -1; }
    if (tid < (DBW ? 2 : 1) * (CM_KC / 8))
        *reinterpret_cast<uint4*>(&sA[(tid >> 3) * WBUF + ZROW * CM_LDA + (tid & 7) * 8]) = make_uint4(0, 0, 0, 0);
    __syncthreads();

    // ---- the tile's slice of N, its row range, and the LDS row of every entry
    {
        // The tile's N rows are contiguous: BM * TAPS consecutive ints, all
        // loads issued before any is used.
        constexpr int NE = (BM * TAPS + 255) / 256;
        const int64_t base = k0 * TAPS;
        const int64_t lim = static_cast<int64_t>(n) * TAPS;
        int m[NE];
#pragma unroll
        for (int u = 0; u < NE; ++u) {
            const int e = tid + 256 * u;
            const bool ok = e < BM * TAPS && base + e < lim;
            const int v = Nt[min(base + min(e, BM * TAPS - 1), lim - 1)];   // clamped: branch-free
            m[u] = ok ? v : -1;
        }
        int lo = 0x7fffffff, hi = -1;
#pragma unroll
        for (int u = 0; u < NE; ++u) {
            const int e = tid + 256 * u;
            const int v = clamp_index(m[u], n);
            if (e < BM * TAPS) sN[e] = v;
            if (v >= 0) { lo = min(lo, v); hi = max(hi, v); }
        }
        // Reduce within the wave first (same-address LDS atomics from every
        // thread serialise), then one atomic pair per wave.
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            lo = min(lo, __shfl_xor(lo, d, 64));
            hi = max(hi, __shfl_xor(hi, d, 64));
        }
        if (lane == 0 && hi >= 0) { atomicMin(&sLo, lo); atomicMax(&sHi, hi); }
    }
    __syncthreads();
    const int wlo = sLo;
    const int span = (sHi >= 0) ? sHi - wlo + 1 : 0;
    const bool window = span <= WIN;
    for (int e = tid; e < BM * TAPS; e += 256) {
        const int m = sN[e];
        sRow[e] = static_cast<short>(m < 0 ? ZROW : (window ? m - wlo : e / TAPS));
    }

    // ---- staging helpers: raw buffer loads, 16-byte pieces.  Pieces outside
    // the tile (rows past the window, output channels past NO, channels past
    // K in a 32-channel tail chunk, -1 entries in gather mode) get an
    // out-of-range offset and read as zeros, so every store below is plain
    // and no load sits behind a branch.
    const rsrc_t rA = make_rsrc(A, static_cast<uint32_t>(n) * K * 2);
    const rsrc_t rB = make_rsrc(B, static_cast<uint32_t>(TAPS) * NO * K * 2);
    auto kc_of = [&](int c) { return min(CM_KC, K - c * CM_KC); };
    auto load_window = [&](int c, uint4* regs) {
        const int c0 = c * CM_KC, kc = kc_of(c);
#pragma unroll
        for (int u = 0; u < WREGS; ++u) {
            const int q = tid + 256 * u;
            const int r = q >> 3, ch = q & 7;
            const bool ok = r < span && ch * 8 < kc;
            regs[u] = load16(rA, ok ? (static_cast<uint32_t>(wlo + r) * K + c0 + ch * 8) * 2 : kOob);
        }
    };
    auto store_window = [&](const uint4* regs, int buf) {
#pragma unroll
        for (int u = 0; u < WREGS; ++u) {
            const int q = tid + 256 * u;
            const int r = q >> 3, ch = q & 7;     // r < WIN: rows past span hold zeros
            *reinterpret_cast<uint4*>(&sA[buf * WBUF + r * CM_LDA + ch * 8]) = regs[u];
        }
    };
    // Weight tile of round rr (chunk rr / TAPS, tap rr % TAPS): B[P-j][n0 + nn][c0 + ...],
    // loaded straight into LDS (buffer_load ... lds: lane L of an
    // instruction writes the 16 bytes at the instruction's LDS base + 16 L),
    // so it needs no registers and no LDS store instructions.  Row nn's
    // 16-byte chunk ch sits at position ch ^ ((nn >> 1) & 7) of its 128-byte
    // row.  LDS serves a 16-byte read 16 lanes at a time over 64 banks (256
    // bytes); the fragment reads of 16 consecutive rows then cover all 64
    // banks once (row parity picks the 128-byte half, the swizzle the 16-byte
    // slot within it).  Each wave issues 4 of the tile's 16 instructions;
    // the lane chooses the chunk that belongs in its slot.  The per-lane part
    // of the offset is fixed; a round adds a uniform part.
    uint32_t bOff[4];
    int bChunk[4];
    {
        const int pos = lane & 7, rsub = lane >> 3;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int nn = (wave * 4 + u) * 8 + rsub;
            bChunk[u] = pos ^ ((nn >> 1) & 7);
            bOff[u] = n0 + nn < NO ? (static_cast<uint32_t>(n0 + nn) * K + bChunk[u] * 8) * 2 : kOob;
        }
    }
    typedef __attribute__((address_space(3))) void lds_void_t;
    auto issue_B = [&](int rr, int buf) {
        const int c = rr / TAPS, j = rr - c * TAPS;
        const int c0 = c * CM_KC, kc = kc_of(c);
        const uint32_t roff = (static_cast<uint32_t>(TAPS - 1 - j) * NO * K + c0) * 2;
        uint16_t* sb = sB[buf];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void_t*)(sb + (wave * 4 + u) * 512), 16,
                                                     bChunk[u] * 8 < kc ? bOff[u] + roff : kOob, 0, 0, 0);
    };
    // Gather mode: the BM rows of tap j, chunk c, straight into sA.
    auto stage_gather = [&](int rr) {
        const int c = rr / TAPS, j = rr - c * TAPS;
        const int c0 = c * CM_KC, kc = kc_of(c);
#pragma unroll
        for (int u = 0; u < BM / 32; ++u) {
            const int q = tid + 256 * u;
            const int r = q >> 3, ch = q & 7;
            const int m = sN[r * TAPS + j];
            const bool ok = m >= 0 && ch * 8 < kc;
            *reinterpret_cast<uint4*>(&sA[r * CM_LDA + ch * 8]) =
                load16(rA, ok ? (static_cast<uint32_t>(m) * K + c0 + ch * 8) * 2 : kOob);
        }
    };

    floatx16_t acc[MB][2];
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = zero16();

    uint4 wreg[WREGS];
    if (window && span > 0) {
        load_window(0, wreg);
        store_window(wreg, 0);
    }
    issue_B(0, 0);
    __syncthreads();                      // also waits for the direct loads

    for (int r = 0; r < R; ++r) {
        const int c = r / TAPS, j = r - c * TAPS;
        if (!window) {
            stage_gather(r);
            __syncthreads();
        }
        // The next round's weights go into the other buffer (last read in
        // round r - 1, before the previous barrier), issued ahead of this
        // round's MFMAs; the barrier at the end of the round waits for them.
        // Mid-chunk, the next chunk's window rows go out first.
        if (window && span > 0 && j == TAPS / 2 && c + 1 < nchunks) load_window(c + 1, wreg);
        if (r + 1 < R) issue_B(r + 1, (r + 1) & 1);
        int arow[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) arow[mb] = sRow[(wm * 32 * MB + mb * 32 + l32) * TAPS + j];
        // Always the full 4 k-steps: a 32-channel tail chunk is zero-filled
        // past its end in both operands, and one code path keeps the
        // accumulators in fixed registers.
        mma_round<MB>(sA + (DBW && window ? (c & 1) * WBUF : 0), sB[r & 1], arow, acc);
        if (r + 1 < R) {
            if (DBW) {
                // the other window buffer was last read in round r - 1,
                // before the previous barrier
                if (window && span > 0) store_window(wreg, (c + 1) & 1);
            } else if (window && span > 0 && (r + 1) % TAPS == 0) {
                __syncthreads();           // every wave is done with this chunk's window
                store_window(wreg, 0);
            }
            __syncthreads();
        }
    }

    // ---- epilogue.  Without a residual: bias, round to bf16, stage the
    // BM x 128 tile in LDS (the first wave row's BM / 2 rows over the window,
    // the second's over the weight buffers), then write whole 16-byte row
    // pieces.
    constexpr int OLD = CM_BN + 8;      // 272-byte pitch: rows 4 apart in opposite bank halves
    constexpr int HALF = BM / 2;
    static_assert(HALF * OLD <= (DBW ? 2 : 1) * WBUF && HALF * OLD <= 2 * CM_SB,
                  "output tile halves must fit the window and the weight buffers");
    uint16_t* const sOutLo = sA;
    uint16_t* const sOutHi = &sB[0][0];
    if (!RES) {
        __syncthreads();
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int cl = wn * 64 + nb * 32 + l32;
            const float bv = (bias && n0 + cl < NO) ? bf16_to_f32(bias[n0 + cl]) : 0.f;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        (wm ? sOutHi : sOutLo)[(mb * 32 + g * 8 + lhi * 4 + q) * OLD + cl] =
                            f32_to_bf16(acc[mb][nb][g * 4 + q] + bv);
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < (BM * CM_BN / 8) / 256; ++u) {
            const int q = tid + 256 * u;
            const int rl = q >> 4, ch = q & 15;
            const int64_t row = k0 + rl;
            const int col = n0 + ch * 8;
            const bool hi = rl >= HALF;
            if (row < n && col < NO)
                *reinterpret_cast<uint4*>(out + row * NO + col) =
                    *reinterpret_cast<const uint4*>(&(hi ? sOutHi : sOutLo)[(rl - (hi ? HALF : 0)) * OLD + ch * 8]);
        }
        return;
    }
    // With a residual: the fp32 sums (bias included) are staged in LDS a
    // quarter tile per region (pass mb holds rows wm*64 + mb*32 .. +31 of
    // both halves: wm = 0 over the window, wm = 1 over the weight buffers),
    // and every thread then adds 16-byte pieces of the residual row and
    // writes 16-byte pieces of the output, rounding once.  The residual
    // pieces are requested before the first barrier (rows past n read as
    // zero through an out-of-range offset; NO % 16 == 0 keeps every piece
    // wholly inside or outside the row).
    constexpr int OLF = CM_BN + 8;      // 544-byte pitch: rows 4 apart 32 banks apart
    static_assert(32 * OLF * 4 <= (DBW ? 2 : 1) * WBUF * 2 && 32 * OLF * 4 <= 2 * CM_SB * 2,
                  "an fp32 quarter tile must fit the window and the weight buffers");
    float* const fLo = reinterpret_cast<float*>(sA);
    float* const fHi = reinterpret_cast<float*>(&sB[0][0]);
    const rsrc_t rR = make_rsrc(res, static_cast<uint32_t>(n) * NO * 2);
    uint4 rres[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int q = tid + 256 * u;
            const int h = q >> 9, r = (q >> 4) & 31, ch = q & 15;
            const int64_t row = k0 + h * 64 + mb * 32 + r;
            const int col = n0 + ch * 8;
            rres[mb][u] = load16(rR, (row < n && col < NO) ? static_cast<uint32_t>((row * NO + col) * 2) : kOob);
        }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        __syncthreads();                // the rounds (mb = 0) or the previous pass's reads are done
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int cl = wn * 64 + nb * 32 + l32;
            const float bv = (bias && n0 + cl < NO) ? bf16_to_f32(bias[n0 + cl]) : 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                (wm ? fHi : fLo)[((e >> 2) * 8 + lhi * 4 + (e & 3)) * OLF + cl] = acc[mb][nb][e] + bv;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int q = tid + 256 * u;
            const int h = q >> 9, r = (q >> 4) & 31, ch = q & 15;
            const int64_t row = k0 + h * 64 + mb * 32 + r;
            const int col = n0 + ch * 8;
            const float* src = (h ? fHi : fLo) + r * OLF + ch * 8;
            const float4 a = *reinterpret_cast<const float4*>(src);
            const float4 b = *reinterpret_cast<const float4*>(src + 4);
            const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            const uint32_t w[4] = {rres[mb][u].x, rres[mb][u].y, rres[mb][u].z, rres[mb][u].w};
            uint32_t o[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t lo = f32_to_bf16(v[2 * p] + bf16_to_f32(static_cast<uint16_t>(w[p] & 0xffffu)));
                const uint32_t hi = f32_to_bf16(v[2 * p + 1] + bf16_to_f32(static_cast<uint16_t>(w[p] >> 16)));
                o[p] = lo | (hi << 16);
            }
            if (row < n && col < NO)
                *reinterpret_cast<uint4*>(out + row * NO + col) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
}

// V[P-j][o][i] = Wt[j][i][o]: one C_in x C_out transpose per tap through
// LDS, 32 x 32 tiles (rows padded by one element), 4 elements per thread.
__global__ __launch_bounds__(256) void k_repack_fwd(const uint16_t* __restrict__ Wt, uint16_t* __restrict__ V,
                                                    int Ci, int Co) {
    __shared__ uint16_t t[32][33];
    const int j = blockIdx.z;
    const int i0 = blockIdx.y * 32, o0 = blockIdx.x * 32;
    const uint16_t* src = Wt + static_cast<int64_t>(j) * Ci * Co;
    uint16_t* dst = V + static_cast<int64_t>(gridDim.z - 1 - j) * Co * Ci;
    const int c = threadIdx.x & 31, r0 = threadIdx.x >> 5;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int r = r0 + 8 * u;                  // r: input channel, c: output channel
        t[r][c] = (i0 + r < Ci && o0 + c < Co) ? src[static_cast<int64_t>(i0 + r) * Co + o0 + c] : 0;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int r = r0 + 8 * u;                  // r: output channel, c: input channel
        if (o0 + r < Co && i0 + c < Ci) dst[static_cast<int64_t>(o0 + r) * Ci + i0 + c] = t[c][r];
    }
}

bool conv_mfma_supported(bool dx, int Ci, int Co, int64_t n, int taps) {
    const int K = dx ? Co : Ci, NO = dx ? Ci : Co;
    const bool built = taps == 1 || taps == 9 || taps == 25 || taps == 49;
    // A, the output (and a residual shaped like it) and B within one buffer range
    return built && K > 0 && NO > 0 && K % 32 == 0 && NO % 16 == 0 && n * K * 2 <= kMaxRange &&
           n * NO * 2 <= kMaxRange && static_cast<int64_t>(taps) * NO * K * 2 <= kMaxRange;
}

size_t conv_mfma_fwd_workspace(int Ci, int Co, int taps) {
    return (static_cast<size_t>(taps) * Ci * Co * sizeof(uint16_t) + 255) & ~static_cast<size_t>(255);
}

hipError_t launch_repack_fwd(const uint16_t* Wt, uint16_t* V, int Ci, int Co, int taps, hipStream_t stream,
                             bool allow_frag) {
    // shapes the fragment-order kernel takes get its layout (same size)
    if (allow_frag && conv_bfrag_ok(Ci, Co, taps)) return launch_repack_frag(Wt, V, Ci, Co, taps, false, stream);
    dim3 grid((Co + 31) / 32, (Ci + 31) / 32, taps);
    hipLaunchKernelGGL(k_repack_fwd, grid, dim3(256), 0, stream, Wt, V, Ci, Co);
    return hipGetLastError();
}

template <int TAPS>
static void launch_taps(dim3 grid, hipStream_t stream, const uint16_t* A, const int32_t* N, const uint16_t* B,
                        const uint16_t* bias, const uint16_t* R, uint16_t* out, int n, int K, int NO,
                        const ConvSecond* second) {
    // the residual and paired variants are instantiations of their own: a
    // runtime test changes the code the compiler emits for the main loop
    const ConvSecond none{nullptr, nullptr, nullptr, 0, 0, 0};
    if (second)
        hipLaunchKernelGGL((k_conv_mfma<TAPS, false, true, 2>), grid, dim3(256), 0, stream, A, N, B, bias, nullptr,
                           out, n, K, NO, *second);
    else if (R)
        hipLaunchKernelGGL((k_conv_mfma<TAPS, true, false, 2>), grid, dim3(256), 0, stream, A, N, B, bias, R, out,
                           n, K, NO, none);
    else
        hipLaunchKernelGGL((k_conv_mfma<TAPS, false, false, 2>), grid, dim3(256), 0, stream, A, N, B, bias, R, out,
                           n, K, NO, none);
}

static hipError_t launch_any(dim3 grid, int taps, hipStream_t stream, const uint16_t* A, const int32_t* N,
                             const uint16_t* B, const uint16_t* bias, const uint16_t* R, uint16_t* out, int n,
                             int K, int NO, const ConvSecond* second) {
    switch (taps) {
        case 1: launch_taps<1>(grid, stream, A, N, B, bias, R, out, n, K, NO, second); break;
        case 9: launch_taps<9>(grid, stream, A, N, B, bias, R, out, n, K, NO, second); break;
        case 25: launch_taps<25>(grid, stream, A, N, B, bias, R, out, n, K, NO, second); break;
        case 49: launch_taps<49>(grid, stream, A, N, B, bias, R, out, n, K, NO, second); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

static int64_t conv_tiles(int64_t n, int NO, int bm = CM_BM) {
    return ((n + bm - 1) / bm) * ((NO + CM_BN - 1) / CM_BN);
}

// Row blocks per wave for a plain 3 x 3 call: 3 (192-token tiles) when that
// takes fewer dispatch rounds of the 512 workgroup slots of a 256-CU part
// (two per compute unit) than 128-token tiles, else 2.  A 192-token tile
// costs about 1.25 times a 128-token one (0.83 instead of 1 KB of LDS reads
// per MFMA), so it only pays when it saves a round: at 39,389 tokens and 256
// output channels, 616 tiles (2 rounds) become 412 (1 round).  Depends on
// the arguments only.  Every output element sums the same products in the
// same order either way, so the choice does not change the result.
static int conv_tile_blocks(int64_t n, int NO, int taps) {
    if (taps != 9) return 2;
    constexpr int64_t kSlots = 512;
    const int64_t r2 = (conv_tiles(n, NO, CM_BM) + kSlots - 1) / kSlots;
    const int64_t r3 = (conv_tiles(n, NO, CM_BM3) + kSlots - 1) / kSlots;
    return r3 < r2 ? 3 : 2;
}

hipError_t launch_conv_mfma_pair(const uint16_t* A1, const uint16_t* B1, const uint16_t* bias1, uint16_t* out1,
                                 int K1, int NO1, const uint16_t* A2, const uint16_t* B2, uint16_t* out2, int K2,
                                 int NO2, const int32_t* N, int64_t n, int taps, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t t1 = conv_tiles(n, NO1), t2 = conv_tiles(n, NO2);
    const ConvSecond second{A2, B2, out2, K2, NO2, static_cast<int>(t1)};
    return launch_any(dim3(static_cast<unsigned>(t1 + t2)), taps, stream, A1, N, B1, bias1, nullptr, out1,
                      static_cast<int>(n), K1, NO1, &second);
}

hipError_t launch_conv_mfma_packed(const uint16_t* A, const int32_t* N, const uint16_t* B,
                                   const uint16_t* bias, const uint16_t* R, uint16_t* out, int64_t n, int K,
                                   int NO, int taps, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    if (!R && conv_tile_blocks(n, NO, taps) == 3) {
        const ConvSecond none{nullptr, nullptr, nullptr, 0, 0, 0};
        hipLaunchKernelGGL((k_conv_mfma<9, false, false, 3>), dim3(static_cast<unsigned>(conv_tiles(n, NO, CM_BM3))),
                           dim3(256), 0, stream, A, N, B, bias, nullptr, out, static_cast<int>(n), K, NO, none);
        return hipGetLastError();
    }
    return launch_any(dim3(static_cast<unsigned>(conv_tiles(n, NO))), taps, stream, A, N, B, bias, R, out,
                      static_cast<int>(n), K, NO, nullptr);
}

}  // namespace svc
