// Weight and bias gradients as a split-K reduction over tokens.
//   dW[j][i][o] = sum_k X[N[k,j]][i] dY[k][o]      (a GEMM with M = taps C_in,
//   db[o]       = sum_k dY[k][o]                     N = C_out, K = tokens)
// for a K x K neighbourhood with taps = K * K (9 in the page's 3 x 3 case).
// ("SV-TAD: Native Sparse Convolutions for Efficient Temporal Action
// Detection", Key Design 2 names dedicated backward kernels; the formula is
// the adjoint of the forward sum.)
//
// The token range is cut into slices; each slice writes fp32 partial sums to
// the workspace and a final pass adds the slices in ascending order, so the
// result is bitwise reproducible.  With one slice the partial kernel writes
// dW directly.
//
// The MFMA kernel (bf16, C_in and C_out multiples of 128) is described
// below; other shapes and fp32 use the VALU kernel in conv_valu.hip.
#include "internal.h"
#include "mfma.h"

namespace svc {

hipError_t launch_dw_valu(bool bf16, const void* X, const int32_t* N, const void* dY, float* out,
                          int64_t n, int Ci, int Co, int taps, int slices, int64_t slice_tokens,
                          int direct, int accumulate, hipStream_t stream);

// MFMA kernel.  A unit is one (tap, 128-input-channel tile) pair; units are
// numbered tap-fastest (u = tile * taps + tap) and cut into groups of three,
// the last group padded with empty units.  At 3 x 3 a group is one kernel
// row (taps 3r, 3r+1, 3r+2) of one input tile; at 1 x 1 it is three input
// tiles.  Workgroup = (group; 128 output channels; token slice), 8 waves.
// Wave w owns input channels 32 (w & 3) .. +31 of the three units and output
// channels 64 (w >> 2) .. +63: 3 x 2 blocks of 32 x 32 (96 accumulators), so
// each dY fragment feeds three units.  An empty unit stages zeros and stores
// nothing.
//
// The contraction runs over tokens while both operands are stored with
// channels contiguous.  Each step of 64 tokens is staged transposed: the
// workgroup's 512 8 x 8 blocks (3 units x 8 token groups x 16 channel groups
// of gathered X rows, 8 x 16 of dY rows; one per thread) are loaded as
// 16-byte rows (the X rows through N[k][unit's tap]), transposed in registers
// and written to LDS channel-major, [tile][channel][token], where every MFMA
// fragment is one 16-byte read.  At the start of step s the tiles of step
// s + 1 go into the free LDS buffer and the row loads of step s + 2 are
// issued, ahead of step s's MFMAs; each step ends with a single barrier.
//
// The N entries a step needs (64 tokens x 3 units) are fetched once per
// workgroup by one wave, lane = token, two steps ahead, and passed through a
// small double-buffered LDS table: per-thread loads would request each entry
// 16 times and touch 8 cache lines per instruction for 32 useful bytes.
//
// All global reads are raw buffer loads with 32-bit offsets: rows of pruned
// neighbours and tokens past the slice get an out-of-range offset and read
// as zeros without a memory request or a branch.  The host sends inputs
// larger than the buffer range (2 GiB) to the VALU kernel.
constexpr int DW_BI = 128, DW_BO = 128, DW_TK = 64, DW_THREADS = 512;
constexpr int DW_LD = DW_TK + 8;                 // 144-byte rows
constexpr int DW_TILE = 128 * DW_LD;             // one [128 channels][64 tokens] tile
constexpr int DW_BUF = 4 * DW_TILE;              // 3 X tiles + 1 dY tile
constexpr int DW_NTAB = 2 * 3 * DW_TK;           // N table: [2 buffers][3 units][64 tokens]
constexpr size_t DW_LDS = 2 * DW_BUF * sizeof(uint16_t) + DW_NTAB * sizeof(int);

__global__ __launch_bounds__(DW_THREADS) void k_dw_mfma(const uint16_t* __restrict__ X,
                                                        const int32_t* __restrict__ Nt,
                                                        const uint16_t* __restrict__ dY,
                                                        float* __restrict__ out, float* __restrict__ dbout,
                                                        int n, int Ci, int Co, int taps, int slice_tokens,
                                                        int direct, int accumulate) {
    extern __shared__ __align__(16) uint16_t dwsm[];   // 2 buffers of DW_BUF, then the N table
    int* const ntab = reinterpret_cast<int*>(dwsm + 2 * DW_BUF);

    // 1-D grid of tiles x slices: logical id = slice * tiles + tile, so the
    // tiles of one token slice (which gather the same X and dY rows) sit
    // together on one XCD and share its L2.
    const int units = taps * (Ci / DW_BI);
    const int groups = (units + 2) / 3;
    const int tiles = groups * (Co / DW_BO);
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int slice = logical / tiles;
    const int bid = logical % tiles;
    const int grp = bid % groups;
    const int o0 = (bid / groups) * DW_BO;
    const int kbeg = slice * slice_tokens;
    const int cnt = max(0, min(n - kbeg, slice_tokens));     // tokens of this slice
    const int steps = (cnt + DW_TK - 1) / DW_TK;
    // one group per output tile also sums db (group 1 at 3 x 3: kernel row 1
    // of the first input tile)
    const bool do_db = dbout != nullptr && grp == min(1, groups - 1);

    // The wave index is uniform across a wave; reading it through the scalar
    // unit lets every per-wave condition below compile to a scalar branch.
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, lhi = lane >> 5;
    const int wi = wave & 3, wo = wave >> 2;

    // This thread's 8 x 8 block: tile = wave >> 1 (units 0..2 of the group,
    // then dY), token group tid & 7, channel group (tid >> 3) & 15.  The block
    // lands at LDS rows cg*8 + e, column tg*8: bank group (tg + e) mod 8 with
    // the 144-byte pitch, so the 8 lanes that share a write cycle (8 token
    // groups) never collide.
    const int tile = wave >> 1, tg = tid & 7, cg = (tid >> 3) & 15;
    const bool is_x = tile < 3;
    // this wave's unit (X tiles only): its tap and input-channel tile
    const int unit = 3 * grp + (is_x ? tile : 0);
    const bool xlive = is_x && unit < units;
    const int utap = unit % taps, ui0 = (unit / taps) * DW_BI;
    const uint32_t nrow = static_cast<uint32_t>(taps) * 4;   // bytes per N row
    const rsrc_t rX = make_rsrc(X, static_cast<uint32_t>(n) * Ci * 2);
    const rsrc_t rN = make_rsrc(Nt + static_cast<int64_t>(kbeg) * taps, static_cast<uint32_t>(cnt) * nrow);
    const rsrc_t rY = make_rsrc(dY + static_cast<int64_t>(kbeg) * Co, static_cast<uint32_t>(cnt) * Co * 2);
    const uint32_t nOff = static_cast<uint32_t>(tg * 8) * nrow + utap * 4;
    const uint32_t yOff = static_cast<uint32_t>(tg * 8) * Co * 2 + (o0 + cg * 8) * 2;
    const uint32_t xCol = (ui0 + cg * 8) * 2, rowX = Ci * 2, rowY = Co * 2;
    uint4 rr[8];
    int ni[8];
    // N entries are used as they are loaded and tested only when the rows
    // they point to are requested: a test right after a load would make the
    // wave wait for it (and for the row loads queued before it) on the spot.
    //   load_n: this thread's 8 entries straight from N (first two steps);
    //   fetch_n / put_n: the loader wave's 3 entries (lane = token) into the
    //     table buffer of the step's parity;
    //   get_n: this thread's 8 entries from the table.
    const bool loader = wave == 6;
    int nreg[3];
    // the loader's column of N for each unit of the group (-1: empty unit)
    int ltap[3];
#pragma unroll
    for (int t = 0; t < 3; ++t) ltap[t] = 3 * grp + t < units ? (3 * grp + t) % taps : -1;
    auto load_n = [&](int s) {
        if (is_x) {
            const uint32_t base = nOff + static_cast<uint32_t>(s * DW_TK) * nrow;
#pragma unroll
            for (int t = 0; t < 8; ++t) ni[t] = load4(rN, base + t * nrow);
        }
    };
    auto fetch_n = [&](int s) {
        const uint32_t base = static_cast<uint32_t>(s * DW_TK + lane) * nrow;
#pragma unroll
        for (int t = 0; t < 3; ++t) nreg[t] = ltap[t] >= 0 ? load4(rN, base + ltap[t] * 4) : -1;
    };
    auto put_n = [&](int s) {
#pragma unroll
        for (int t = 0; t < 3; ++t) ntab[((s & 1) * 3 + t) * DW_TK + lane] = nreg[t];
    };
    auto get_n = [&](int s) {
        const int* p = &ntab[((s & 1) * 3 + tile) * DW_TK + tg * 8];
        const int4 a = *reinterpret_cast<const int4*>(p), b = *reinterpret_cast<const int4*>(p + 4);
        ni[0] = a.x; ni[1] = a.y; ni[2] = a.z; ni[3] = a.w;
        ni[4] = b.x; ni[5] = b.y; ni[6] = b.z; ni[7] = b.w;
    };
    auto load_rows = [&](int s) {
        if (is_x) {
            const int lim = cnt - s * DW_TK - tg * 8;     // tokens t < lim lie in the slice
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const bool ok = xlive && static_cast<unsigned>(ni[t]) < static_cast<unsigned>(n) && t < lim;
                rr[t] = load16(rX, ok ? __umul24(static_cast<unsigned>(ni[t]), rowX) + xCol : kOob);
            }
        } else {
            const uint32_t base = yOff + static_cast<uint32_t>(s * DW_TK) * rowY;
#pragma unroll
            for (int t = 0; t < 8; ++t) rr[t] = load16(rY, base + t * rowY);   // past the slice: zeros
        }
    };
    auto store_rows = [&](int buf) {
        uint16_t* sb = dwsm + buf * DW_BUF + tile * DW_TILE;
        uint4 c[8];
        transpose8x8_b16(rr, c);
#pragma unroll
        for (int e = 0; e < 8; ++e) *reinterpret_cast<uint4*>(&sb[(cg * 8 + e) * DW_LD + tg * 8]) = c[e];
    };

    floatx16_t acc[3][2];
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[t][b] = zero16();
    // db: thread = (output channel o0 + (tid & 127), 16-token quarter tid >> 7)
    // of each step's dY tile, summed with bf16 dot products against ones.
    float dbacc = 0.f;
    typedef __attribute__((__vector_size__(2 * sizeof(short)))) short short2_t;
    const short2_t ones = __builtin_bit_cast(short2_t, 0x3f803f80u);

    if (steps > 0) {
        load_n(0);
        load_rows(0);
        store_rows(0);
        if (steps > 1) { load_n(1); load_rows(1); }
        if (loader && steps > 2) {
            fetch_n(2);
            put_n(2);
            if (steps > 3) fetch_n(3);
        }
    }
    __syncthreads();

    // One step.  With `all` every look-ahead exists (s + 4 < steps): the
    // main loop runs that form without any branch around loads and stores,
    // so the compiler's wait counts stay exact; the last steps take the
    // guarded form.
    auto step = [&](int s, bool all) {
        const bool n1 = all || s + 1 < steps, n2 = all || s + 2 < steps;
        const bool n3 = all || s + 3 < steps, n4 = all || s + 4 < steps;
        // Step s + 2's N entries from the table (written in step s - 1), the
        // next step's tiles into the free buffer (last read in step s - 1),
        // the loader wave's table entries for step s + 3 (into the buffer
        // step s + 1 read in step s - 1) and the row loads of step s + 2:
        // all ahead of this step's MFMAs.  The loader's entries go out
        // before the row loads, so that neither waits behind the other.
        if (is_x && n2) get_n(s + 2);
        if (n1) store_rows((s + 1) & 1);
        if (loader && n3) {
            put_n(s + 3);
            if (n4) fetch_n(s + 4);
        }
        if (n2) load_rows(s + 2);
        const uint16_t* __restrict__ sb = dwsm + (s & 1) * DW_BUF;
        const uint16_t* __restrict__ sd = sb + 3 * DW_TILE;
#pragma unroll
        for (int ks = 0; ks < DW_TK / 16; ++ks) {
            const int kof = ks * 16 + lhi * 8;
            bf16x8_t a[3], b[2];
#pragma unroll
            for (int t = 0; t < 3; ++t) a[t] = frag_row(&sb[t * DW_TILE + (wi * 32 + l32) * DW_LD + kof]);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) b[nb] = frag_row(&sd[(wo * 64 + nb * 32 + l32) * DW_LD + kof]);
#pragma unroll
            for (int t = 0; t < 3; ++t)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) acc[t][nb] = mfma32(a[t], b[nb], acc[t][nb]);
        }
        if (do_db) {
            const uint16_t* p = &sd[(tid & 127) * DW_LD + (tid >> 7) * 16];
            const uint4 v0 = *reinterpret_cast<const uint4*>(p);
            const uint4 v1 = *reinterpret_cast<const uint4*>(p + 8);
            const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int h = 0; h < 8; ++h)
                dbacc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(short2_t, w[h]), ones, dbacc, false);
        }
        if (n1) __syncthreads();
    };
    int s = 0;
    for (; s + 4 < steps; ++s) step(s, true);
    for (; s < steps; ++s) step(s, false);

    // D block (32 input channels x 32 output channels): lane holds output
    // channel l32 and input channels 8g + 4*lhi + q.
    float* dst = out + (direct ? 0 : static_cast<int64_t>(slice) * taps * Ci * Co);
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        const int u = 3 * grp + t;
        if (u >= units) continue;
        const int i0 = (u / taps) * DW_BI;
        float* dj = dst + static_cast<int64_t>(u % taps) * Ci * Co;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int i = i0 + wi * 32 + g * 8 + lhi * 4 + q;
                    const int o = o0 + wo * 64 + nb * 32 + l32;
                    float* d = dj + static_cast<int64_t>(i) * Co + o;
                    const float v = acc[t][nb][g * 4 + q];
                    *d = (direct && accumulate) ? *d + v : v;
                }
    }
    if (do_db) {
        // the four quarters of each channel, added in a fixed order
        float* red = reinterpret_cast<float*>(dwsm);
        __syncthreads();
        red[tid] = dbacc;
        __syncthreads();
        if (tid < DW_BO) {
            const float v = ((red[tid] + red[tid + 128]) + red[tid + 256]) + red[tid + 384];
            float* d = dbout + (direct ? 0 : static_cast<int64_t>(slice) * Co) + o0 + tid;
            *d = (direct && accumulate) ? *d + v : v;
        }
    }
}

// db partials: block = 64 columns x 4 row phases; fixed-order combine in LDS.
template <typename T>
__global__ __launch_bounds__(256) void k_db_partial(const T* __restrict__ dY, float* __restrict__ part,
                                                    int n, int Co, int64_t slice_tokens) {
    __shared__ float red[4][64];
    const int c = threadIdx.x & 63, ph = threadIdx.x >> 6;
    const int o = blockIdx.x * 64 + c;
    const int64_t kbeg = static_cast<int64_t>(blockIdx.y) * slice_tokens;
    const int64_t kend = min(static_cast<int64_t>(n), kbeg + slice_tokens);
    float sum = 0.f;
    if (o < Co)
        for (int64_t k = kbeg + ph; k < kend; k += 4) sum += Elem<T>::load(dY + k * Co + o);
    red[ph][c] = sum;
    __syncthreads();
    if (ph == 0 && o < Co)
        part[static_cast<int64_t>(blockIdx.y) * Co + o] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
}

// out[e] (+)= sum_{s < slices} part[s][e], s ascending (4 floats per thread).
// The db partials ride along: block 0 also reduces them (Co floats, one per
// thread, same order), which saves a launch.
__global__ __launch_bounds__(256) void k_reduce_slices4(const float4* __restrict__ part, float4* __restrict__ out,
                                                        int64_t count4, int slices, int accumulate,
                                                        const float* __restrict__ dbpart, float* __restrict__ db,
                                                        int Co) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < count4; e += stride) {
        // loads issued 8 slices at a time (one wait per batch instead of one
        // per slice), added in slice order
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        int s = 0;
        for (; s + 8 <= slices; s += 8) {
            float4 p[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) p[u] = part[static_cast<int64_t>(s + u) * count4 + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                v.x += p[u].x; v.y += p[u].y; v.z += p[u].z; v.w += p[u].w;
            }
        }
        for (; s < slices; ++s) {
            const float4 p = part[static_cast<int64_t>(s) * count4 + e];
            v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
        }
        if (accumulate) {
            const float4 o = out[e];
            v.x = o.x + v.x; v.y = o.y + v.y; v.z = o.z + v.z; v.w = o.w + v.w;
        }
        out[e] = v;
    }
    if (db && blockIdx.x == 0)
        for (int o = threadIdx.x; o < Co; o += blockDim.x) {
            // loads issued 8 at a time, added in slice order
            float v = 0.f;
            int s = 0;
            for (; s + 8 <= slices; s += 8) {
                float p[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) p[u] = dbpart[static_cast<int64_t>(s + u) * Co + o];
#pragma unroll
                for (int u = 0; u < 8; ++u) v += p[u];
            }
            for (; s < slices; ++s) v += dbpart[static_cast<int64_t>(s) * Co + o];
            db[o] = accumulate ? db[o] + v : v;
        }
}

// out[e] (+)= sum_{s < slices} part[s][e], s ascending.
__global__ __launch_bounds__(256) void k_reduce_slices(const float* __restrict__ part, float* __restrict__ out,
                                                       int64_t count, int slices, int accumulate) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < count; e += stride) {
        float v = 0.f;
        int s = 0;
        for (; s + 8 <= slices; s += 8) {
            float p[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) p[u] = part[static_cast<int64_t>(s + u) * count + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) v += p[u];
        }
        for (; s < slices; ++s) v += part[static_cast<int64_t>(s) * count + e];
        out[e] = accumulate ? out[e] + v : v;
    }
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

DwPlan plan_dw(int64_t n, int Ci, int Co, bool bf16, int taps) {
    DwPlan p{};
    p.taps = taps;
    // The MFMA kernel addresses X, dY and N through 32-bit buffer offsets.
    p.mfma = bf16 && Ci % DW_BI == 0 && Co % DW_BO == 0 && n * Ci * 2 <= kMaxRange &&
             n * Co * 2 <= kMaxRange && n * taps * 4 <= kMaxRange;
    int64_t slices;
    const int64_t step = p.mfma ? DW_TK : 16;
    if (p.mfma) {
        // Split-K factor from a small cost model: one workgroup per compute
        // unit of a 256-CU part at ~4 TFLOP/s, counted in whole dispatch
        // rounds, plus the fp32 partials written and read back (~5 TB/s) and
        // a fixed cost for the extra reduction launch.  Depends on the
        // arguments only, so workspace sizing and the call agree.
        const int64_t tiles = ceil_div(static_cast<int64_t>(taps) * (Ci / DW_BI), 3) * (Co / DW_BO);
        const double flops = 2.0 * static_cast<double>(n) * static_cast<double>(3 * tiles / (Co / DW_BO)) * DW_BI * Co;
        const double dwb = static_cast<double>(taps) * Ci * Co * 4;
        double best = 1e30;
        slices = 1;
        for (int64_t s = 1; s <= 64; ++s) {
            if (s > 1 && ceil_div(n, s) < 4 * DW_TK) break;
            const double rounds = static_cast<double>(ceil_div(tiles * s, 256));
            const double t = rounds * flops / static_cast<double>(tiles * s) / 4e12 +
                             (s > 1 ? (2.0 * static_cast<double>(s) * dwb / 5e12 + 4e-6) : 0.0);
            if (t < best) { best = t; slices = s; }
        }
    } else {
        const int64_t tiles = static_cast<int64_t>(taps) * ceil_div(Ci, 64) * ceil_div(Co, 64);
        slices = ceil_div(512, tiles);
        slices = std::min<int64_t>(slices, std::max<int64_t>(1, n / 512));
        slices = std::max<int64_t>(1, std::min<int64_t>(slices, 64));
    }
    int64_t st = ceil_div(std::max<int64_t>(n, 1), slices);
    st = ceil_div(st, step) * step;
    slices = std::max<int64_t>(1, ceil_div(n, st));
    p.slices = static_cast<int>(slices);
    p.slice_tokens = st;
    p.partial_floats = slices > 1 ? static_cast<size_t>(slices) * taps * Ci * Co : 0;
    p.db_floats = static_cast<size_t>(slices) * Co;
    return p;
}

size_t dw_workspace_bytes(const DwPlan& p) {
    auto up = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
    return up(p.partial_floats * sizeof(float)) + up(p.db_floats * sizeof(float));
}

// Phase 1: the partial kernels (dW straight into dW with one slice, else
// the slices' partials into the workspace; db partials likewise).
hipError_t launch_dw_partials(const DwPlan& plan, bool bf16, const void* X, const int32_t* N, const void* dY,
                              float* dW, float* db, int64_t n, int Ci, int Co, int accumulate, void* ws,
                              hipStream_t stream) {
    auto up = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
    float* part = static_cast<float*>(ws);
    float* dbpart = reinterpret_cast<float*>(static_cast<char*>(ws) + up(plan.partial_floats * sizeof(float)));
    const bool direct = plan.slices == 1;
    hipError_t err;
    if (plan.mfma) {
        // 145.5 KiB of dynamic LDS: above the default limit, so raise it once.
        static const hipError_t attr = hipFuncSetAttribute(
            reinterpret_cast<const void*>(k_dw_mfma), hipFuncAttributeMaxDynamicSharedMemorySize,
            static_cast<int>(DW_LDS));
        if (attr != hipSuccess) return attr;
        const int groups = (plan.taps * (Ci / DW_BI) + 2) / 3;
        dim3 grid(groups * (Co / DW_BO) * plan.slices);
        hipLaunchKernelGGL(k_dw_mfma, grid, dim3(DW_THREADS), DW_LDS, stream, static_cast<const uint16_t*>(X), N,
                           static_cast<const uint16_t*>(dY), direct ? dW : part,
                           db ? (direct ? db : dbpart) : nullptr, static_cast<int>(n), Ci, Co, plan.taps,
                           static_cast<int>(plan.slice_tokens), direct ? 1 : 0, accumulate);
        return hipGetLastError();
    }
    err = launch_dw_valu(bf16, X, N, dY, direct ? dW : part, n, Ci, Co, plan.taps, plan.slices,
                         plan.slice_tokens, direct ? 1 : 0, accumulate, stream);
    if (err != hipSuccess || !db) return err;
    dim3 grid(static_cast<unsigned>(ceil_div(Co, 64)), plan.slices);
    if (bf16)
        hipLaunchKernelGGL(k_db_partial<uint16_t>, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(dY),
                           dbpart, static_cast<int>(n), Co, plan.slice_tokens);
    else
        hipLaunchKernelGGL(k_db_partial<float>, grid, dim3(256), 0, stream, static_cast<const float*>(dY), dbpart,
                           static_cast<int>(n), Co, plan.slice_tokens);
    return hipGetLastError();
}

// Phase 2: the fixed-order reduction of whatever phase 1 left in the
// workspace (nothing with one slice on the MFMA path).
hipError_t launch_dw_reduce(const DwPlan& plan, float* dW, float* db, int Ci, int Co, int accumulate,
                            const void* ws, hipStream_t stream) {
    auto up = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
    const float* part = static_cast<const float*>(ws);
    const float* dbpart =
        reinterpret_cast<const float*>(static_cast<const char*>(ws) + up(plan.partial_floats * sizeof(float)));
    const bool direct = plan.slices == 1;
    hipError_t err = hipSuccess;
    // db partials of the MFMA kernel go through the dW reduction launch.
    bool db_done = db && plan.mfma && direct;
    if (!direct) {
        const int64_t count = static_cast<int64_t>(plan.taps) * Ci * Co;
        if (count % 4 == 0) {
            const int blocks = static_cast<int>(std::min<int64_t>(ceil_div(count / 4, 256), 8192));
            hipLaunchKernelGGL(k_reduce_slices4, dim3(blocks), dim3(256), 0, stream,
                               reinterpret_cast<const float4*>(part), reinterpret_cast<float4*>(dW), count / 4,
                               plan.slices, accumulate, db ? dbpart : nullptr, db, Co);
            db_done = db != nullptr;
        } else {
            const int blocks = static_cast<int>(std::min<int64_t>(ceil_div(count, 256), 8192));
            hipLaunchKernelGGL(k_reduce_slices, dim3(blocks), dim3(256), 0, stream, part, dW, count,
                               plan.slices, accumulate);
        }
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (db && !db_done) {
        const int blocks = static_cast<int>(ceil_div(Co, 256));
        hipLaunchKernelGGL(k_reduce_slices, dim3(blocks), dim3(256), 0, stream, dbpart, db,
                           static_cast<int64_t>(Co), plan.slices, accumulate);
        err = hipGetLastError();
    }
    return err;
}

hipError_t launch_dw(const DwPlan& plan, bool bf16, const void* X, const int32_t* N, const void* dY,
                     float* dW, float* db, int64_t n, int Ci, int Co, int accumulate, void* ws,
                     hipStream_t stream) {
    hipError_t err = launch_dw_partials(plan, bf16, X, N, dY, dW, db, n, Ci, Co, accumulate, ws, stream);
    if (err != hipSuccess) return err;
    return launch_dw_reduce(plan, dW, db, Ci, Co, accumulate, ws, stream);
}

}  // namespace svc
