// Weight and bias gradients as a split-K reduction over tokens.
//   dW[j][i][o] = sum_k X[N[k,j]][i] dY[k][o]      (a GEMM with M = 9 C_in,
//   db[o]       = sum_k dY[k][o]                     N = C_out, K = tokens)
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
                          int64_t n, int Ci, int Co, int slices, int64_t slice_tokens, int direct,
                          int accumulate, hipStream_t stream);

// MFMA kernel: workgroup = (kernel row r: taps 3r, 3r+1, 3r+2; 128 input
// channels; 128 output channels; token slice), 8 waves.  Wave w owns input
// channels 32 (w & 3) .. +31 for the three taps and output channels
// 64 (w >> 2) .. +63: 3 x 2 blocks of 32 x 32 (96 accumulators), so each dY
// fragment feeds three taps.
//
// The contraction runs over tokens while both operands are stored with
// channels contiguous.  Each step of 64 tokens is staged transposed: the
// workgroup's 512 8 x 8 blocks (3 taps x 8 token groups x 16 channel groups
// of gathered X rows, 8 x 16 of dY rows; one per thread) are loaded as
// 16-byte rows (the X rows through N[k][3r + tap]), transposed in registers
// and written to LDS channel-major, [tile][channel][token], where every MFMA
// fragment is one 16-byte read.  At the start of step s the tiles of step
// s + 1 go into the free LDS buffer and the loads of step s + 2 (N entries of
// step s + 3) are issued, ahead of step s's MFMAs; each step ends with a
// single barrier.
constexpr int DW_BI = 128, DW_BO = 128, DW_TK = 64, DW_THREADS = 512;
constexpr int DW_LD = DW_TK + 8;                 // 144-byte rows
constexpr int DW_TILE = 128 * DW_LD;             // one [128 channels][64 tokens] tile
constexpr int DW_BUF = 4 * DW_TILE;              // 3 X tiles + 1 dY tile

__global__ __launch_bounds__(DW_THREADS) void k_dw_mfma(const uint16_t* __restrict__ X,
                                                        const int32_t* __restrict__ Nt,
                                                        const uint16_t* __restrict__ dY,
                                                        float* __restrict__ out, float* __restrict__ dbout,
                                                        int n, int Ci, int Co, int64_t slice_tokens,
                                                        int direct, int accumulate) {
    extern __shared__ __align__(16) uint16_t dwsm[];   // 2 buffers of DW_BUF

    // 1-D grid of tiles x slices: logical id = slice * tiles + tile, so the
    // tiles of one token slice (which gather the same X and dY rows) sit
    // together on one XCD and share its L2.
    const int tilesI = Ci / DW_BI;
    const int tiles = 3 * tilesI * (Co / DW_BO);
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int slice = logical / tiles;
    int bid = logical % tiles;
    const int kr = bid % 3;
    bid /= 3;
    const int i0 = (bid % tilesI) * DW_BI;
    const int o0 = (bid / tilesI) * DW_BO;
    const int64_t kbeg = static_cast<int64_t>(slice) * slice_tokens;
    const int64_t kend = min(static_cast<int64_t>(n), kbeg + slice_tokens);
    const int steps = kend > kbeg ? static_cast<int>((kend - kbeg + DW_TK - 1) / DW_TK) : 0;
    const bool do_db = dbout != nullptr && kr == 1 && i0 == 0;

    // The wave index is uniform across a wave; reading it through the scalar
    // unit lets every per-wave condition below compile to a scalar branch.
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, lhi = lane >> 5;
    const int wi = wave & 3, wo = wave >> 2;

    // This thread's 8 x 8 block: tile = tid >> 7 (taps 0..2 of the row, then
    // dY), token group tid & 7, channel group (tid >> 3) & 15.  The block
    // lands at LDS rows cg*8 + e, column tg*8: bank group (tg + e) mod 8 with
    // the 144-byte pitch, so the 8 lanes that share a write cycle (8 token
    // groups) never collide.
    const int tile = wave >> 1, tg = tid & 7, cg = (tid >> 3) & 15;
    const bool is_x = tile < 3;
    uint4 rr[8];
    int ni[8];
    // Loads of pruned neighbours are masked off (no memory request at all):
    // the gathered X rows are the kernel's main traffic.
    const int64_t klast = kend - 1;
    const int ncol = 3 * kr + (is_x ? tile : 0);
    // The N entries are loaded unconditionally (clamped address) and only
    // tested when the rows they point to are requested, one step later: a
    // test right after the load would make the wave wait for it, and for the
    // row loads queued before it.
    auto load_n = [&](int s) {
        const int64_t kb = kbeg + static_cast<int64_t>(s) * DW_TK + tg * 8;
        if (is_x)
#pragma unroll
            for (int t = 0; t < 8; ++t) ni[t] = Nt[min(kb + t, klast) * 9 + ncol];
    };
    auto load_rows = [&](int s) {
        const int64_t kb = kbeg + static_cast<int64_t>(s) * DW_TK + tg * 8;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (is_x) {
                const int j = clamp_index(ni[t], n);
                if (j >= 0 && kb + t <= klast)
                    v = *reinterpret_cast<const uint4*>(X + static_cast<int64_t>(j) * Ci + i0 + cg * 8);
            } else {
                const int64_t k = kb + t;
                if (k <= klast) v = *reinterpret_cast<const uint4*>(dY + k * Co + o0 + cg * 8);
            }
            rr[t] = v;
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
    float dbacc = 0.f;

    if (steps > 0) {
        load_n(0);
        load_rows(0);
        store_rows(0);
        if (steps > 1) { load_n(1); load_rows(1); }
        if (steps > 2) load_n(2);
    }
    __syncthreads();

    for (int s = 0; s < steps; ++s) {
        // Next step's tiles into the free buffer (last read in step s - 1),
        // loads for the step after, N entries for the one after that: all
        // issued ahead of this step's MFMAs.
        if (s + 1 < steps) {
            store_rows((s + 1) & 1);
            if (s + 2 < steps) load_rows(s + 2);
            if (s + 3 < steps) load_n(s + 3);
        }
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
        if (do_db && wave < DW_BO / 64) {
            // row tid of the dY tile: output channel o0 + tid over the 64 tokens
#pragma unroll
            for (int q = 0; q < DW_TK / 8; ++q) {
                const uint4 v = *reinterpret_cast<const uint4*>(&sd[tid * DW_LD + q * 8]);
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    dbacc += bf16_to_f32(static_cast<uint16_t>(w[h] & 0xffffu));
                    dbacc += bf16_to_f32(static_cast<uint16_t>(w[h] >> 16));
                }
            }
        }
        if (s + 1 < steps) __syncthreads();
    }

    // D block (32 input channels x 32 output channels): lane holds output
    // channel l32 and input channels 8g + 4*lhi + q.
    float* dst = out + (direct ? 0 : static_cast<int64_t>(slice) * 9 * Ci * Co);
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        float* dj = dst + static_cast<int64_t>(3 * kr + t) * Ci * Co;
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
    if (do_db && wave < DW_BO / 64) {
        float* d = dbout + (direct ? 0 : static_cast<int64_t>(slice) * Co) + o0 + tid;
        *d = (direct && accumulate) ? *d + dbacc : dbacc;
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
__global__ __launch_bounds__(256) void k_reduce_slices4(const float4* __restrict__ part, float4* __restrict__ out,
                                                        int64_t count4, int slices, int accumulate) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < count4; e += stride) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s = 0; s < slices; ++s) {
            const float4 p = part[static_cast<int64_t>(s) * count4 + e];
            v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
        }
        if (accumulate) {
            const float4 o = out[e];
            v.x = o.x + v.x; v.y = o.y + v.y; v.z = o.z + v.z; v.w = o.w + v.w;
        }
        out[e] = v;
    }
}

// out[e] (+)= sum_{s < slices} part[s][e], s ascending.
__global__ __launch_bounds__(256) void k_reduce_slices(const float* __restrict__ part, float* __restrict__ out,
                                                       int64_t count, int slices, int accumulate) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < count; e += stride) {
        float v = 0.f;
        for (int s = 0; s < slices; ++s) v += part[static_cast<int64_t>(s) * count + e];
        out[e] = accumulate ? out[e] + v : v;
    }
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

DwPlan plan_dw(int64_t n, int Ci, int Co, bool bf16) {
    DwPlan p{};
    p.mfma = bf16 && Ci % DW_BI == 0 && Co % DW_BO == 0;
    int64_t slices;
    const int64_t step = p.mfma ? DW_TK : 16;
    if (p.mfma) {
        // Split-K factor from a small cost model: one workgroup per compute
        // unit of a 256-CU part at ~4 TFLOP/s, counted in whole dispatch
        // rounds, plus the fp32 partials written and read back (~5 TB/s) and
        // a fixed cost for the extra reduction launch.  Depends on the
        // arguments only, so workspace sizing and the call agree.
        const int64_t tiles = 3ll * (Ci / DW_BI) * (Co / DW_BO);
        const double flops = 2.0 * static_cast<double>(n) * 9 * Ci * Co;
        const double dwb = 9.0 * Ci * Co * 4;
        double best = 1e30;
        slices = 1;
        for (int64_t s = 1; s <= 64; ++s) {
            if (s > 1 && ceil_div(n, s) < 4 * DW_TK) break;
            const double rounds = static_cast<double>(ceil_div(tiles * s, 256));
            const double t = rounds * flops / static_cast<double>(tiles * s) / 4e12 +
                             (s > 1 ? (2.0 * s * dwb / 5e12 + 4e-6) : 0.0);
            if (t < best) { best = t; slices = s; }
        }
    } else {
        const int64_t tiles = 9ll * ceil_div(Ci, 64) * ceil_div(Co, 64);
        slices = ceil_div(512, tiles);
        slices = std::min<int64_t>(slices, std::max<int64_t>(1, n / 512));
        slices = std::max<int64_t>(1, std::min<int64_t>(slices, 64));
    }
    int64_t st = ceil_div(std::max<int64_t>(n, 1), slices);
    st = ceil_div(st, step) * step;
    slices = std::max<int64_t>(1, ceil_div(n, st));
    p.slices = static_cast<int>(slices);
    p.slice_tokens = st;
    p.partial_floats = slices > 1 ? static_cast<size_t>(slices) * 9 * Ci * Co : 0;
    p.db_floats = static_cast<size_t>(slices) * Co;
    return p;
}

size_t dw_workspace_bytes(const DwPlan& p) {
    auto up = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
    return up(p.partial_floats * sizeof(float)) + up(p.db_floats * sizeof(float));
}

hipError_t launch_dw(const DwPlan& plan, bool bf16, const void* X, const int32_t* N, const void* dY,
                     float* dW, float* db, int64_t n, int Ci, int Co, int accumulate, void* ws,
                     hipStream_t stream) {
    auto up = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
    float* part = static_cast<float*>(ws);
    float* dbpart = reinterpret_cast<float*>(static_cast<char*>(ws) + up(plan.partial_floats * sizeof(float)));
    const bool direct = plan.slices == 1;
    hipError_t err;
    if (plan.mfma) {
        // 144 KiB of dynamic LDS: above the default limit, so raise it once.
        static const hipError_t attr = hipFuncSetAttribute(
            reinterpret_cast<const void*>(k_dw_mfma), hipFuncAttributeMaxDynamicSharedMemorySize,
            static_cast<int>(2 * DW_BUF * sizeof(uint16_t)));
        if (attr != hipSuccess) return attr;
        dim3 grid(3 * (Ci / DW_BI) * (Co / DW_BO) * plan.slices);
        hipLaunchKernelGGL(k_dw_mfma, grid, dim3(DW_THREADS), 2 * DW_BUF * sizeof(uint16_t), stream, static_cast<const uint16_t*>(X), N,
                           static_cast<const uint16_t*>(dY), direct ? dW : part,
                           db ? (direct ? db : dbpart) : nullptr, static_cast<int>(n), Ci, Co,
                           plan.slice_tokens, direct ? 1 : 0, accumulate);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    } else {
        err = launch_dw_valu(bf16, X, N, dY, direct ? dW : part, n, Ci, Co, plan.slices, plan.slice_tokens,
                             direct ? 1 : 0, accumulate, stream);
        if (err != hipSuccess) return err;
        if (db) {
            dim3 grid(static_cast<unsigned>(ceil_div(Co, 64)), plan.slices);
            if (bf16)
                hipLaunchKernelGGL(k_db_partial<uint16_t>, grid, dim3(256), 0, stream,
                                   static_cast<const uint16_t*>(dY), dbpart, static_cast<int>(n), Co,
                                   plan.slice_tokens);
            else
                hipLaunchKernelGGL(k_db_partial<float>, grid, dim3(256), 0, stream,
                                   static_cast<const float*>(dY), dbpart, static_cast<int>(n), Co,
                                   plan.slice_tokens);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
    }
    if (!direct) {
        const int64_t count = 9ll * Ci * Co;
        if (count % 4 == 0) {
            const int blocks = static_cast<int>(std::min<int64_t>(ceil_div(count / 4, 256), 8192));
            hipLaunchKernelGGL(k_reduce_slices4, dim3(blocks), dim3(256), 0, stream,
                               reinterpret_cast<const float4*>(part), reinterpret_cast<float4*>(dW), count / 4,
                               plan.slices, accumulate);
        } else {
            const int blocks = static_cast<int>(std::min<int64_t>(ceil_div(count, 256), 8192));
            hipLaunchKernelGGL(k_reduce_slices, dim3(blocks), dim3(256), 0, stream, part, dW, count,
                               plan.slices, accumulate);
        }
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (db && !(plan.mfma && direct)) {
        const int blocks = static_cast<int>(ceil_div(Co, 256));
        hipLaunchKernelGGL(k_reduce_slices, dim3(blocks), dim3(256), 0, stream, dbpart, db,
                           static_cast<int64_t>(Co), plan.slices, accumulate);
        err = hipGetLastError();
    }
    return err;
}

}  // namespace svc
