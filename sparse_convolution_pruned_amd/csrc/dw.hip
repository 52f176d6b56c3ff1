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
// MFMA kernel (bf16, C_in and C_out multiples of 128): workgroup = (tap j,
// 128 input channels, 128 output channels, token slice), 4 waves of 64 x 64.
// The contraction runs over tokens, but both operands are stored token-major
// with channels contiguous; each staging step therefore loads 64 tokens x 8
// channels per thread as 8 x 16-byte rows (the X rows gathered through
// N[k][j]), transposes the 8 x 8 block in registers and writes it to LDS
// channel-major, where every MFMA lane finds its 8 consecutive tokens in one
// 16-byte read.
#include "internal.h"

namespace svc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

hipError_t launch_dw_valu(bool bf16, const void* X, const int32_t* N, const void* dY, float* out,
                          int64_t n, int Ci, int Co, int slices, int64_t slice_tokens, int direct,
                          int accumulate, hipStream_t stream);

constexpr int DW_BI = 128, DW_BO = 128, DW_TK = 64, DW_LD = DW_TK + 8;

__global__ __launch_bounds__(256) void k_dw_mfma(const uint16_t* __restrict__ X,
                                                 const int32_t* __restrict__ Nt,
                                                 const uint16_t* __restrict__ dY,
                                                 float* __restrict__ out, int n, int Ci, int Co,
                                                 int64_t slice_tokens, int direct, int accumulate) {
    __shared__ __align__(16) uint16_t sG[DW_BI * DW_LD];
    __shared__ __align__(16) uint16_t sD[DW_BO * DW_LD];

    const int tilesI = Ci / DW_BI;
    int bid = blockIdx.x;
    const int j = bid % 9;
    bid /= 9;
    const int i0 = (bid % tilesI) * DW_BI;
    const int o0 = (bid / tilesI) * DW_BO;
    const int64_t kbeg = static_cast<int64_t>(blockIdx.y) * slice_tokens;
    const int64_t kend = min(static_cast<int64_t>(n), kbeg + slice_tokens);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int s = tid & 127, tg = s >> 4, cg = s & 15;   // staging: token group, channel group
    const bool stage_g = tid < 128;

    floatx4_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    for (int64_t kb = kbeg; kb < kend; kb += DW_TK) {
        uint4 rows[8], cols[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int64_t k = kb + tg * 8 + r;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (k < kend) {
                if (stage_g) {
                    const int m = clamp_index(Nt[k * 9 + j], n);
                    if (m >= 0) v = *reinterpret_cast<const uint4*>(X + static_cast<int64_t>(m) * Ci + i0 + cg * 8);
                } else {
                    v = *reinterpret_cast<const uint4*>(dY + k * Co + o0 + cg * 8);
                }
            }
            rows[r] = v;
        }
        transpose8x8_b16(rows, cols);
        uint16_t* dst = stage_g ? sG : sD;
        __syncthreads();   // previous step's MFMA reads are done
#pragma unroll
        for (int e = 0; e < 8; ++e)
            *reinterpret_cast<uint4*>(&dst[(cg * 8 + e) * DW_LD + tg * 8]) = cols[e];
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < DW_TK; ks += 32) {
            const int kof = ks + (lane >> 4) * 8;
            bf16x8_t a[4], b[4];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
                a[mb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                                                         &sG[(wm * 64 + mb * 16 + (lane & 15)) * DW_LD + kof]));
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
                b[nb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                                                         &sD[(wn * 64 + nb * 16 + (lane & 15)) * DW_LD + kof]));
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb], b[nb], acc[mb][nb], 0, 0, 0);
        }
    }

    float* dst = out + (direct ? static_cast<int64_t>(j) * Ci * Co
                               : (static_cast<int64_t>(blockIdx.y) * 9 + j) * Ci * Co);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = i0 + wm * 64 + mb * 16 + (lane >> 4) * 4 + q;
                const int o = o0 + wn * 64 + nb * 16 + (lane & 15);
                float* d = dst + static_cast<int64_t>(i) * Co + o;
                *d = (direct && accumulate) ? *d + acc[mb][nb][q] : acc[mb][nb][q];
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
    const int64_t tiles = p.mfma ? 9ll * (Ci / DW_BI) * (Co / DW_BO)
                                 : 9ll * ceil_div(Ci, 64) * ceil_div(Co, 64);
    const int64_t step = p.mfma ? DW_TK : 16;
    // Aim at ~512 workgroups (two per compute unit of a 256-CU part) while
    // keeping at least 512 tokens in a slice.  The plan depends on the
    // arguments only, so workspace sizing and the call always agree.
    int64_t slices = ceil_div(512, tiles);
    slices = std::min<int64_t>(slices, std::max<int64_t>(1, n / 512));
    slices = std::max<int64_t>(1, std::min<int64_t>(slices, 64));
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
    float* target = direct ? dW : part;
    hipError_t err;
    if (plan.mfma) {
        dim3 grid(9 * (Ci / DW_BI) * (Co / DW_BO), plan.slices);
        hipLaunchKernelGGL(k_dw_mfma, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(X), N,
                           static_cast<const uint16_t*>(dY), target, static_cast<int>(n), Ci, Co,
                           plan.slice_tokens, direct ? 1 : 0, accumulate);
        err = hipGetLastError();
    } else {
        err = launch_dw_valu(bf16, X, N, dY, target, n, Ci, Co, plan.slices, plan.slice_tokens,
                             direct ? 1 : 0, accumulate, stream);
    }
    if (err != hipSuccess) return err;
    if (!direct) {
        const int64_t count = 9ll * Ci * Co;
        const int blocks = static_cast<int>(std::min<int64_t>(ceil_div(count, 256), 4096));
        hipLaunchKernelGGL(k_reduce_slices, dim3(blocks), dim3(256), 0, stream, part, dW, count,
                           plan.slices, accumulate);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
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
        const int blocks = static_cast<int>(ceil_div(Co, 256));
        hipLaunchKernelGGL(k_reduce_slices, dim3(blocks), dim3(256), 0, stream, dbpart, db,
                           static_cast<int64_t>(Co), plan.slices, accumulate);
        err = hipGetLastError();
    }
    return err;
}

}  // namespace svc
