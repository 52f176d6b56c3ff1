// Gather-FMA kernels on the vector ALUs: any channel count, fp32 or bf16
// storage, fp32 accumulation.  ("SV-TAD: Native Sparse Convolutions for
// Efficient Temporal Action Detection", Key Design 2: for narrow channel
// counts the gather of neighbour features and the product run in one launch.)
//
// Any odd K x K neighbourhood: `taps` = K * K columns of N, weights
// [taps][C_in][C_out], and tap taps-1-j mirrors tap j.
//
// Forward / input gradient: one workgroup per 64 tokens x 64 output channels.
// The tile's 64 x taps slice of N is read once into LDS; then, tap by tap, 16
// channels at a time, the gathered neighbour rows and the matching weight
// slice are staged in LDS (as fp32) and every thread accumulates a 4 x 4 block
// of outputs with FMAs.  A tap whose entry is -1 stages zeros (zero padding).
// An optional residual R [n][channels produced] is added before the store.
//
// Weight gradient: one workgroup per (tap, 64 input channels, 64 output
// channels, token slice); 16 tokens at a time the gathered X rows and the dY
// rows are staged in LDS and each thread accumulates a 4 x 4 block of dW.
#include "internal.h"

namespace svc {

constexpr int VT_M = 64, VT_N = 64, VT_K = 16;

template <typename T, bool DX>
__global__ __launch_bounds__(256) void k_conv_valu(const T* __restrict__ A,
                                                   const int32_t* __restrict__ Nt,
                                                   const T* __restrict__ Wt,
                                                   const T* __restrict__ bias,
                                                   const T* __restrict__ R,
                                                   T* __restrict__ out, int n, int Ci, int Co, int taps) {
    // K: channels contracted per tap; NO: channels produced.
    const int K = DX ? Co : Ci;
    const int NO = DX ? Ci : Co;
    __shared__ float sA[VT_K][VT_M + 4];
    __shared__ float sB[VT_K][VT_N + 4];
    extern __shared__ int sN[];              // [VT_M][taps], dynamic

    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int64_t k0 = static_cast<int64_t>(blockIdx.x) * VT_M;
    const int n0 = blockIdx.y * VT_N;

    for (int e = tid; e < VT_M * taps; e += 256) {
        const int64_t k = k0 + e / taps;
        sN[e] = (k < n) ? clamp_index(Nt[k * taps + e % taps], n) : -1;
    }
    float acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;
    __syncthreads();

    for (int j = 0; j < taps; ++j) {
        // Input gradient: the row gathered through tap j meets weight tap
        // taps-1-j.
        const int jt = DX ? taps - 1 - j : j;
        const T* __restrict__ Wj = Wt + static_cast<int64_t>(jt) * Ci * Co;
        for (int c0 = 0; c0 < K; c0 += VT_K) {
            for (int e = tid; e < VT_M * VT_K; e += 256) {
                const int r = e / VT_K, kk = e % VT_K;
                const int m = sN[r * taps + j];
                float v = 0.f;
                if (m >= 0 && c0 + kk < K) v = Elem<T>::load(A + static_cast<int64_t>(m) * K + c0 + kk);
                sA[kk][r] = v;
            }
            for (int e = tid; e < VT_K * VT_N; e += 256) {
                float v = 0.f;
                if (!DX) {
                    const int kk = e / VT_N, nn = e % VT_N;
                    if (c0 + kk < K && n0 + nn < NO)
                        v = Elem<T>::load(Wj + static_cast<int64_t>(c0 + kk) * Co + n0 + nn);
                    sB[kk][nn] = v;
                } else {
                    // B(o, i) = Wt[taps-1-j][i][o]: read along o (contiguous).
                    const int nn = e / VT_K, kk = e % VT_K;
                    if (c0 + kk < K && n0 + nn < NO)
                        v = Elem<T>::load(Wj + static_cast<int64_t>(n0 + nn) * Co + c0 + kk);
                    sB[kk][nn] = v;
                }
            }
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < VT_K; ++kk) {
                float a[4], b[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    a[q] = sA[kk][ty + 16 * q];
                    b[q] = sB[kk][tx + 16 * q];
                }
#pragma unroll
                for (int p = 0; p < 4; ++p)
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[p][q] = fmaf(a[p], b[q], acc[p][q]);
            }
            __syncthreads();
        }
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int64_t row = k0 + ty + 16 * p;
        if (row >= n) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int col = n0 + tx + 16 * q;
            if (col >= NO) continue;
            float v = acc[p][q];
            if (!DX && bias) v += Elem<T>::load(bias + col);
            if (R) v += Elem<T>::load(R + row * NO + col);
            Elem<T>::store(out + row * NO + col, v);
        }
    }
}

hipError_t launch_conv_valu(bool bf16, bool dx, const void* A, const int32_t* N, const void* Wt,
                            const void* bias, const void* R, void* out, int64_t n, int Ci, int Co, int taps,
                            hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const size_t lds = static_cast<size_t>(VT_M) * taps * sizeof(int);
    const int NO = dx ? Ci : Co;
    dim3 grid(static_cast<unsigned>((n + VT_M - 1) / VT_M), static_cast<unsigned>((NO + VT_N - 1) / VT_N));
    const int nn = static_cast<int>(n);
    if (bf16) {
        auto a = static_cast<const uint16_t*>(A);
        auto w = static_cast<const uint16_t*>(Wt);
        auto b = static_cast<const uint16_t*>(bias);
        auto r = static_cast<const uint16_t*>(R);
        auto o = static_cast<uint16_t*>(out);
        if (dx) hipLaunchKernelGGL((k_conv_valu<uint16_t, true>), grid, dim3(256), lds, stream, a, N, w, b, r, o, nn, Ci, Co, taps);
        else hipLaunchKernelGGL((k_conv_valu<uint16_t, false>), grid, dim3(256), lds, stream, a, N, w, b, r, o, nn, Ci, Co, taps);
    } else {
        auto a = static_cast<const float*>(A);
        auto w = static_cast<const float*>(Wt);
        auto b = static_cast<const float*>(bias);
        auto r = static_cast<const float*>(R);
        auto o = static_cast<float*>(out);
        if (dx) hipLaunchKernelGGL((k_conv_valu<float, true>), grid, dim3(256), lds, stream, a, N, w, b, r, o, nn, Ci, Co, taps);
        else hipLaunchKernelGGL((k_conv_valu<float, false>), grid, dim3(256), lds, stream, a, N, w, b, r, o, nn, Ci, Co, taps);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------- dW
template <typename T>
__global__ __launch_bounds__(256) void k_dw_valu(const T* __restrict__ X,
                                                 const int32_t* __restrict__ Nt,
                                                 const T* __restrict__ dY, float* __restrict__ out,
                                                 int n, int Ci, int Co, int taps, int64_t slice_tokens,
                                                 int direct, int accumulate) {
    __shared__ float sG[VT_K][VT_M + 4];
    __shared__ float sD[VT_K][VT_N + 4];
    const int tilesI = (Ci + VT_M - 1) / VT_M;
    const int i0 = (blockIdx.x % tilesI) * VT_M;
    const int o0 = (blockIdx.x / tilesI) * VT_N;
    const int j = blockIdx.y;
    const int64_t kbeg = static_cast<int64_t>(blockIdx.z) * slice_tokens;
    const int64_t kend = min(static_cast<int64_t>(n), kbeg + slice_tokens);
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    float acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;

    for (int64_t kb = kbeg; kb < kend; kb += VT_K) {
        for (int e = tid; e < VT_K * VT_M; e += 256) {
            const int kk = e / VT_M, c = e % VT_M;
            const int64_t k = kb + kk;
            float g = 0.f, d = 0.f;
            if (k < kend) {
                const int m = clamp_index(Nt[k * taps + j], n);
                if (m >= 0 && i0 + c < Ci) g = Elem<T>::load(X + static_cast<int64_t>(m) * Ci + i0 + c);
                if (o0 + c < Co) d = Elem<T>::load(dY + k * Co + o0 + c);
            }
            sG[kk][c] = g;
            sD[kk][c] = d;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < VT_K; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                a[q] = sG[kk][ty + 16 * q];
                b[q] = sD[kk][tx + 16 * q];
            }
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[p][q] = fmaf(a[p], b[q], acc[p][q]);
        }
        __syncthreads();
    }
    float* dst = out + (direct ? static_cast<int64_t>(j) * Ci * Co
                               : (static_cast<int64_t>(blockIdx.z) * taps + j) * Ci * Co);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int i = i0 + ty + 16 * p;
        if (i >= Ci) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int o = o0 + tx + 16 * q;
            if (o >= Co) continue;
            float* d = dst + static_cast<int64_t>(i) * Co + o;
            *d = (direct && accumulate) ? *d + acc[p][q] : acc[p][q];
        }
    }
}

hipError_t launch_dw_valu(bool bf16, const void* X, const int32_t* N, const void* dY, float* out,
                          int64_t n, int Ci, int Co, int taps, int slices, int64_t slice_tokens,
                          int direct, int accumulate, hipStream_t stream) {
    const int tiles = ((Ci + VT_M - 1) / VT_M) * ((Co + VT_N - 1) / VT_N);
    dim3 grid(tiles, taps, slices);
    if (bf16)
        hipLaunchKernelGGL(k_dw_valu<uint16_t>, grid, dim3(256), 0, stream,
                           static_cast<const uint16_t*>(X), N, static_cast<const uint16_t*>(dY), out,
                           static_cast<int>(n), Ci, Co, taps, slice_tokens, direct, accumulate);
    else
        hipLaunchKernelGGL(k_dw_valu<float>, grid, dim3(256), 0, stream,
                           static_cast<const float*>(X), N, static_cast<const float*>(dY), out,
                           static_cast<int>(n), Ci, Co, taps, slice_tokens, direct, accumulate);
    return hipGetLastError();
}

}  // namespace svc
