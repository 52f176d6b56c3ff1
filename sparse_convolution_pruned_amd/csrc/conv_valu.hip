// Gather-FMA kernels on the vector ALUs: any channel count, fp32 or bf16
// storage, fp32 accumulation.  ("SV-TAD: Native Sparse Convolutions for
// Efficient Temporal Action Detection", Key Design 2: for narrow channel
// counts the gather of neighbour features and the product run in one launch.)
//
// Any odd K x K neighbourhood: `taps` = K * K columns of N, weights
// [taps][C_in][C_out], and tap taps-1-j mirrors tap j.
//
// Forward / input gradient: one workgroup per 128 tokens x 64 output
// channels.  The tile's 128 x taps slice of N is read once into LDS; then, tap
// by tap, 16 channels at a time, the gathered neighbour rows and the matching
// weight slice are staged in LDS (as fp32) and every thread accumulates an
// 8 x 4 block of outputs with FMAs.  A tap whose entry is -1 stages zeros
// (zero padding).  An optional residual R [n][channels produced] is added
// before the store.
//
// Weight gradient: one workgroup per (tap, 64 input channels, 64 output
// channels, token slice); 16 tokens at a time the gathered X rows and the dY
// rows are staged in LDS and each thread accumulates a 4 x 4 block of dW.
#include <type_traits>

#include "internal.h"

namespace svc {

// Weight-gradient tile.
constexpr int VT_M = 64, VT_N = 64, VT_K = 16;

// Four consecutive elements from global memory as fp32 (VEC: one 16- or
// 8-byte load; the caller checks alignment and range).
template <typename T> struct Vec4;
template <> struct Vec4<float> {
    static __device__ __forceinline__ void load(const float* p, float* v) {
        const float4 x = *reinterpret_cast<const float4*>(p);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    }
};
template <> struct Vec4<uint16_t> {
    static __device__ __forceinline__ void load(const uint16_t* p, float* v) {
        const uint2 x = *reinterpret_cast<const uint2*>(p);
        v[0] = bf16_to_f32(static_cast<uint16_t>(x.x & 0xffffu));
        v[1] = bf16_to_f32(static_cast<uint16_t>(x.x >> 16));
        v[2] = bf16_to_f32(static_cast<uint16_t>(x.y & 0xffffu));
        v[3] = bf16_to_f32(static_cast<uint16_t>(x.y >> 16));
    }
};

// Forward / input-gradient tile: FT_M tokens x FT_N produced channels per
// workgroup of 256 threads, FT_K contracted channels per round (one tap j, one
// chunk of channels c0).  Thread (ty, tx) owns the 8 x 4 outputs rows
// 8 ty .. 8 ty + 7, columns 4 tx .. 4 tx + 3, read from LDS as 128-bit
// vectors: 12 floats per 32 FMAs (a 4 x 4 block reads 8 per 16, and then the
// LDS rather than the FMA pipes sets the pace).
//
// Rounds are software-pipelined over two LDS buffers: round r + 1's elements
// are loaded into registers while round r's FMAs run, then written to the
// other buffer; one barrier per round.  VEC (channel counts multiples of 4,
// A and the weights aligned to 4 elements): each thread stages four
// consecutive channels with one 16- or 8-byte load.  Every output sums its
// terms in the same order either way: taps, then chunks, then channels.
constexpr int FT_M = 128, FT_N = 64, FT_K = 16;
constexpr int FT_PA = FT_M + 4, FT_PB = FT_N + 4;   // padded LDS rows, multiples of 4 floats

template <typename T, bool DX, bool VEC>
__global__ __launch_bounds__(256) void k_conv_valu(const T* __restrict__ A,
                                                   const int32_t* __restrict__ Nt,
                                                   const T* __restrict__ Wt,
                                                   const T* __restrict__ bias,
                                                   const T* __restrict__ R,
                                                   T* __restrict__ out, int n, int Ci, int Co, int taps) {
    // K: channels contracted per tap; NO: channels produced.
    const int K = DX ? Co : Ci;
    const int NO = DX ? Ci : Co;
    __shared__ __align__(16) float sA[2][FT_K][FT_PA];
    __shared__ __align__(16) float sB[2][FT_K][FT_PB];
    extern __shared__ int sN[];              // [FT_M][taps], dynamic

    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int64_t k0 = static_cast<int64_t>(blockIdx.x) * FT_M;
    const int n0 = blockIdx.y * FT_N;

    for (int e = tid; e < FT_M * taps; e += 256) {
        const int64_t k = k0 + e / taps;
        sN[e] = (k < n) ? clamp_index(Nt[k * taps + e % taps], n) : -1;
    }
    float acc[8][4];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;
    __syncthreads();

    const int nck = (K + FT_K - 1) / FT_K;
    const int rounds = taps * nck;
    // Staged elements of one round, as fp32: A (FT_M x FT_K) 8 per thread,
    // B (FT_K x FT_N) 4 per thread.
    float va[8], vb[4];
    auto fetch = [&](int r) {
        const int j = r / nck, c0 = (r - j * nck) * FT_K;
        // Input gradient: the row gathered through tap j meets weight tap
        // taps-1-j.
        const int jt = DX ? taps - 1 - j : j;
        const T* __restrict__ Wj = Wt + static_cast<int64_t>(jt) * Ci * Co;
        if (VEC) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {   // A: row tid / 4 + 64 i, channels c0 + 4 (tid % 4) ..
                const int row = (tid >> 2) + 64 * i, kq = (tid & 3) * 4;
                const int m = sN[row * taps + j];
                if (m >= 0 && c0 + kq < K) Vec4<T>::load(A + static_cast<int64_t>(m) * K + c0 + kq, va + 4 * i);
                else va[4 * i] = va[4 * i + 1] = va[4 * i + 2] = va[4 * i + 3] = 0.f;
            }
            if (!DX) {   // B(kk, c) = Wj[c0 + kk][n0 + c]: kk = tid / 16, c = 4 (tid % 16) ..
                const int kk = tid >> 4, cq = (tid & 15) * 4;
                if (c0 + kk < K && n0 + cq < NO) Vec4<T>::load(Wj + static_cast<int64_t>(c0 + kk) * Co + n0 + cq, vb);
                else vb[0] = vb[1] = vb[2] = vb[3] = 0.f;
            } else {     // B(kk, c) = Wt[taps-1-j][n0 + c][c0 + kk]: c = tid / 4, kk = 4 (tid % 4) ..
                const int c = tid >> 2, kq = (tid & 3) * 4;
                if (n0 + c < NO && c0 + kq < K) Vec4<T>::load(Wj + static_cast<int64_t>(n0 + c) * Co + c0 + kq, vb);
                else vb[0] = vb[1] = vb[2] = vb[3] = 0.f;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {   // A: row tid / 16 + 16 i, channel c0 + tid % 16
                const int row = (tid >> 4) + 16 * i, kk = tid & 15;
                const int m = sN[row * taps + j];
                va[i] = (m >= 0 && c0 + kk < K) ? Elem<T>::load(A + static_cast<int64_t>(m) * K + c0 + kk) : 0.f;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (!DX) {   // kk = tid / 64 + 4 i, c = tid % 64
                    const int kk = (tid >> 6) + 4 * i, c = tid & 63;
                    vb[i] = (c0 + kk < K && n0 + c < NO)
                                ? Elem<T>::load(Wj + static_cast<int64_t>(c0 + kk) * Co + n0 + c) : 0.f;
                } else {     // c = tid / 16 + 16 i, kk = tid % 16 (read along Co, contiguous)
                    const int c = (tid >> 4) + 16 * i, kk = tid & 15;
                    vb[i] = (c0 + kk < K && n0 + c < NO)
                                ? Elem<T>::load(Wj + static_cast<int64_t>(n0 + c) * Co + c0 + kk) : 0.f;
                }
            }
        }
    };
    auto commit = [&](int buf) {
        if (VEC) {
            const int kq = (tid & 3) * 4;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) sA[buf][kq + q][(tid >> 2) + 64 * i] = va[4 * i + q];
            if (!DX) {
                *reinterpret_cast<float4*>(&sB[buf][tid >> 4][(tid & 15) * 4]) = make_float4(vb[0], vb[1], vb[2], vb[3]);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) sB[buf][kq + q][tid >> 2] = vb[q];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) sA[buf][tid & 15][(tid >> 4) + 16 * i] = va[i];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (!DX) sB[buf][(tid >> 6) + 4 * i][tid & 63] = vb[i];
                else sB[buf][tid & 15][(tid >> 4) + 16 * i] = vb[i];
            }
        }
    };

    fetch(0);
    commit(0);
    __syncthreads();
    for (int r = 0; r < rounds; ++r) {
        const int cur = r & 1;
        const bool more = r + 1 < rounds;
        if (more) fetch(r + 1);
        const float* __restrict__ pa = &sA[cur][0][8 * ty];
        const float* __restrict__ pb = &sB[cur][0][4 * tx];
        // Unrolled by 2 only: fully unrolled, the compiler issued all 48
        // LDS reads of the round ahead of the FMAs (~250 VGPRs, one wave per
        // SIMD).
#pragma unroll 2
        for (int kk = 0; kk < FT_K; ++kk) {
            const float4 a0 = *reinterpret_cast<const float4*>(pa + kk * FT_PA);
            const float4 a1 = *reinterpret_cast<const float4*>(pa + kk * FT_PA + 4);
            const float4 b = *reinterpret_cast<const float4*>(pb + kk * FT_PB);
            const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int p = 0; p < 8; ++p)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[p][q] = fmaf(av[p], bv[q], acc[p][q]);
        }
        if (more) commit(cur ^ 1);
        __syncthreads();
    }

    const int col = n0 + 4 * tx;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int64_t row = k0 + 8 * ty + p;
        if (row >= n) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (col + q >= NO) continue;
            float v = acc[p][q];
            if (!DX && bias) v += Elem<T>::load(bias + col + q);
            if (R) v += Elem<T>::load(R + row * NO + col + q);
            Elem<T>::store(out + row * NO + col + q, v);
        }
    }
}

// Small problems: one workgroup per 16 tokens x 16 produced channels, one
// output per thread, 64 contracted channels per round, the next round loaded
// into registers while the current one is summed.  A 128 x 64 tile holds one
// workgroup on its compute unit and walks its rounds with each wave waiting
// on its loads, so while the wide tiles number fewer than the compute units
// a pass takes the same time whatever the token count (about 80 us at 64
// channels, 300 us at 256, for 98 tokens as for 16,000).  The small tiles
// spread the same work over 32 times as many workgroups; measured, they win
// up to about 190 wide tiles.  The terms of every output are summed in the
// same order (taps, then channels), so both kernels give the same bits.
//
// Both operands sit in LDS with the contracted index contiguous, so a
// thread reads four channels of its row and of its column with two 128-bit
// reads per four FMAs.  The loads are raw buffer loads: an element out of
// range (a pruned neighbour, a channel or token past the end) gets an offset
// past the buffer's range and reads as zero, with no branch.  Operands above
// 2 GiB go to the wide kernels (host check).  Loading further rounds ahead
// was measured slower.
constexpr int ST_M = 16, ST_N = 16, ST_K = 64, ST_P = ST_K + 4;
constexpr int64_t kValuSmallBelow = 192;    // 128 x 64 tiles under which the small kernel runs

template <typename T> __device__ __forceinline__ uint32_t raw_load(rsrc_t r, uint32_t off);
template <> __device__ __forceinline__ uint32_t raw_load<float>(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
template <> __device__ __forceinline__ uint32_t raw_load<uint16_t>(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
template <typename T> __device__ __forceinline__ float raw_f32(uint32_t v) {
    return __uint_as_float(sizeof(T) == 2 ? v << 16 : v);
}
// acc += a[0] b[0] + ... + a[3] b[3], one term at a time in that order.
__device__ __forceinline__ float fma4(const float4 a, const float4 b, float acc) {
    acc = fmaf(a.x, b.x, acc);
    acc = fmaf(a.y, b.y, acc);
    acc = fmaf(a.z, b.z, acc);
    return fmaf(a.w, b.w, acc);
}

template <typename T, bool DX>
__global__ __launch_bounds__(256) void k_conv_valu_small(const T* __restrict__ A, const int32_t* __restrict__ Nt,
                                                         const T* __restrict__ Wt, const T* __restrict__ bias,
                                                         const T* __restrict__ R, T* __restrict__ out, int n, int Ci,
                                                         int Co, int taps) {
    constexpr uint32_t es = sizeof(T);
    const int K = DX ? Co : Ci;
    const int NO = DX ? Ci : Co;
    const rsrc_t rA = make_rsrc(A, static_cast<uint32_t>(static_cast<int64_t>(n) * K * es));
    const rsrc_t rW = make_rsrc(Wt, static_cast<uint32_t>(static_cast<int64_t>(taps) * Ci * Co * es));
    __shared__ __align__(16) float sA[2][ST_M][ST_P];     // [row][channel]
    __shared__ __align__(16) float sB[2][ST_N][ST_P];     // [column][channel]
    extern __shared__ int sN[];                           // [ST_M][taps], dynamic
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int64_t k0 = static_cast<int64_t>(blockIdx.x) * ST_M;
    const int n0 = blockIdx.y * ST_N;
    for (int e = tid; e < ST_M * taps; e += 256) {
        const int64_t k = k0 + e / taps;
        sN[e] = (k < n) ? clamp_index(Nt[k * taps + e % taps], n) : -1;
    }
    __syncthreads();

    const int nck = (K + ST_K - 1) / ST_K;
    const int rounds = taps * nck;
    // Round r: A (16 rows x 64 channels) and B (64 channels x 16 columns),
    // four elements of each per thread, held raw until written to LDS.
    uint32_t va[4], vb[4];
    auto fetch = [&](int r) {
        const int j = r / nck, c0 = (r - j * nck) * ST_K;
        const int jt = DX ? taps - 1 - j : j;        // input gradient: the mirrored weight tap
        const uint32_t wj = static_cast<uint32_t>(jt) * Ci * Co;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + 256 * i;
            const int row = e >> 6, kk = e & 63;
            const int m = sN[row * taps + j];
            va[i] = raw_load<T>(rA, (m >= 0 && c0 + kk < K) ? (static_cast<uint32_t>(m) * K + c0 + kk) * es : kOob);
            int kb, c;
            uint32_t w;
            if (!DX) {   // B(kb, c) = Wt[j][c0 + kb][n0 + c]
                kb = e >> 4;
                c = e & 15;
                w = wj + static_cast<uint32_t>(c0 + kb) * Co + n0 + c;
            } else {     // B(kb, c) = Wt[taps-1-j][n0 + c][c0 + kb], read along Co
                c = e >> 6;
                kb = e & 63;
                w = wj + static_cast<uint32_t>(n0 + c) * Co + c0 + kb;
            }
            vb[i] = raw_load<T>(rW, (c0 + kb < K && n0 + c < NO) ? w * es : kOob);
        }
    };
    auto commit = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + 256 * i;
            sA[buf][e >> 6][e & 63] = raw_f32<T>(va[i]);
            if (!DX) sB[buf][e & 15][e >> 4] = raw_f32<T>(vb[i]);
            else sB[buf][e >> 6][e & 63] = raw_f32<T>(vb[i]);
        }
    };
    fetch(0);
    commit(0);
    __syncthreads();
    float acc = 0.f;
    for (int r = 0; r < rounds; ++r) {
        const int cur = r & 1;
        const bool more = r + 1 < rounds;
        if (more) fetch(r + 1);
        const float* __restrict__ a = &sA[cur][ty][0];
        const float* __restrict__ bb = &sB[cur][tx][0];
#pragma unroll 4
        for (int kk = 0; kk < ST_K; kk += 4)
            acc = fma4(*reinterpret_cast<const float4*>(a + kk), *reinterpret_cast<const float4*>(bb + kk), acc);
        if (more) commit(cur ^ 1);
        __syncthreads();
    }
    const int64_t row = k0 + ty;
    const int col = n0 + tx;
    if (row < n && col < NO) {
        float v = acc;
        if (!DX && bias) v += Elem<T>::load(bias + col);
        if (R) v += Elem<T>::load(R + row * NO + col);
        Elem<T>::store(out + row * NO + col, v);
    }
}

template <typename T>
static void launch_valu_typed(bool dx, bool vec, dim3 grid, size_t lds, hipStream_t stream, const T* A,
                              const int32_t* N, const T* Wt, const T* bias, const T* R, T* out, int n, int Ci,
                              int Co, int taps) {
    const dim3 block(256);
    if (dx && vec) hipLaunchKernelGGL((k_conv_valu<T, true, true>), grid, block, lds, stream, A, N, Wt, bias, R, out, n, Ci, Co, taps);
    else if (dx) hipLaunchKernelGGL((k_conv_valu<T, true, false>), grid, block, lds, stream, A, N, Wt, bias, R, out, n, Ci, Co, taps);
    else if (vec) hipLaunchKernelGGL((k_conv_valu<T, false, true>), grid, block, lds, stream, A, N, Wt, bias, R, out, n, Ci, Co, taps);
    else hipLaunchKernelGGL((k_conv_valu<T, false, false>), grid, block, lds, stream, A, N, Wt, bias, R, out, n, Ci, Co, taps);
}

hipError_t launch_conv_valu(bool bf16, bool dx, const void* A, const int32_t* N, const void* Wt,
                            const void* bias, const void* R, void* out, int64_t n, int Ci, int Co, int taps,
                            hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const size_t lds = static_cast<size_t>(FT_M) * taps * sizeof(int);
    const int NO = dx ? Ci : Co;
    dim3 grid(static_cast<unsigned>((n + FT_M - 1) / FT_M), static_cast<unsigned>((NO + FT_N - 1) / FT_N));
    const int nn = static_cast<int>(n);
    const int64_t esz = bf16 ? 2 : 4;
    if (static_cast<int64_t>(grid.x) * grid.y < kValuSmallBelow && n * (dx ? Co : Ci) * esz <= kMaxRange &&
        static_cast<int64_t>(taps) * Ci * Co * esz <= kMaxRange) {
        const dim3 sgrid(static_cast<unsigned>((n + ST_M - 1) / ST_M), static_cast<unsigned>((NO + ST_N - 1) / ST_N));
        const size_t slds = static_cast<size_t>(ST_M) * taps * sizeof(int);
#define SV_VALU_SMALL(T)                                                                                              \
    do {                                                                                                              \
        auto a = static_cast<const T*>(A);                                                                            \
        auto w = static_cast<const T*>(Wt);                                                                           \
        auto b = static_cast<const T*>(bias);                                                                         \
        auto r = static_cast<const T*>(R);                                                                            \
        auto o = static_cast<T*>(out);                                                                                \
        if (dx) hipLaunchKernelGGL((k_conv_valu_small<T, true>), sgrid, dim3(256), slds, stream, a, N, w, b, r, o, nn, \
                                   Ci, Co, taps);                                                                     \
        else hipLaunchKernelGGL((k_conv_valu_small<T, false>), sgrid, dim3(256), slds, stream, a, N, w, b, r, o, nn,  \
                                Ci, Co, taps);                                                                        \
    } while (0)
        if (bf16) SV_VALU_SMALL(uint16_t);
        else SV_VALU_SMALL(float);
#undef SV_VALU_SMALL
        return hipGetLastError();
    }
    // four-channel loads: channel counts multiples of 4 and A, Wt aligned to 4 elements
    const size_t es = bf16 ? 2 : 4;
    const bool vec = Ci % 4 == 0 && Co % 4 == 0 && reinterpret_cast<uintptr_t>(A) % (4 * es) == 0 &&
                     reinterpret_cast<uintptr_t>(Wt) % (4 * es) == 0;
    if (bf16)
        launch_valu_typed(dx, vec, grid, lds, stream, static_cast<const uint16_t*>(A), N,
                          static_cast<const uint16_t*>(Wt), static_cast<const uint16_t*>(bias),
                          static_cast<const uint16_t*>(R), static_cast<uint16_t*>(out), nn, Ci, Co, taps);
    else
        launch_valu_typed(dx, vec, grid, lds, stream, static_cast<const float*>(A), N, static_cast<const float*>(Wt),
                          static_cast<const float*>(bias), static_cast<const float*>(R), static_cast<float*>(out),
                          nn, Ci, Co, taps);
    return hipGetLastError();
}

// ------------------------------------------------------------------- dW
template <typename T>
__global__ __launch_bounds__(256) void k_dw_valu(const T* __restrict__ X,
                                                 const int32_t* __restrict__ Nt,
                                                 const T* __restrict__ dY, float* __restrict__ out,
                                                 int n, int Ci, int Co, int taps, int64_t slice_tokens,
                                                 int direct, int accumulate) {
    // Each thread owns 4 consecutive input x 4 consecutive output channels
    // and reads them as one 128-bit LDS read per operand per token.  Rounds
    // of VT_K tokens are double-buffered: round r + 1 is loaded into
    // registers while round r is summed, then written to the other buffer,
    // one barrier per round.  (Plain 64-bit addressing: inputs above 2 GiB
    // come here.)
    __shared__ __align__(16) float sG[2][VT_K][VT_M + 4];
    __shared__ __align__(16) float sD[2][VT_K][VT_N + 4];
    const int tilesI = (Ci + VT_M - 1) / VT_M;
    const int i0 = (blockIdx.x % tilesI) * VT_M;
    const int o0 = (blockIdx.x / tilesI) * VT_N;
    const int j = blockIdx.y;
    const int64_t kbeg = static_cast<int64_t>(blockIdx.z) * slice_tokens;
    const int64_t kend = min(static_cast<int64_t>(n), kbeg + slice_tokens);
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    constexpr int PER = VT_K * VT_M / 256;          // elements of each operand per thread and round
    float vg[PER], vd[PER];
    auto fetch = [&](int64_t kb) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = tid + 256 * u;
            const int kk = e / VT_M, c = e % VT_M;
            const int64_t k = kb + kk;
            float g = 0.f, d = 0.f;
            if (k < kend) {
                const int m = clamp_index(Nt[k * taps + j], n);
                if (m >= 0 && i0 + c < Ci) g = Elem<T>::load(X + static_cast<int64_t>(m) * Ci + i0 + c);
                if (o0 + c < Co) d = Elem<T>::load(dY + k * Co + o0 + c);
            }
            vg[u] = g;
            vd[u] = d;
        }
    };
    auto commit = [&](int buf) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = tid + 256 * u;
            sG[buf][e / VT_M][e % VT_M] = vg[u];
            sD[buf][e / VT_M][e % VT_M] = vd[u];
        }
    };
    float acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;

    if (kbeg < kend) {
        fetch(kbeg);
        commit(0);
    }
    __syncthreads();
    int cur = 0;
    for (int64_t kb = kbeg; kb < kend; kb += VT_K) {
        const bool more = kb + VT_K < kend;
        if (more) fetch(kb + VT_K);
#pragma unroll 4
        for (int kk = 0; kk < VT_K; ++kk) {
            const float4 a4 = *reinterpret_cast<const float4*>(&sG[cur][kk][4 * ty]);
            const float4 b4 = *reinterpret_cast<const float4*>(&sD[cur][kk][4 * tx]);
            const float a[4] = {a4.x, a4.y, a4.z, a4.w}, b[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[p][q] = fmaf(a[p], b[q], acc[p][q]);
        }
        if (more) commit(cur ^ 1);
        __syncthreads();
        cur ^= 1;
    }
    float* dst = out + (direct ? static_cast<int64_t>(j) * Ci * Co
                               : (static_cast<int64_t>(blockIdx.z) * taps + j) * Ci * Co);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int i = i0 + 4 * ty + p;
        if (i >= Ci) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int o = o0 + 4 * tx + q;
            if (o >= Co) continue;
            float* d = dst + static_cast<int64_t>(i) * Co + o;
            *d = (direct && accumulate) ? *d + acc[p][q] : acc[p][q];
        }
    }
}

// Small problems: 16 input x 16 output channels per workgroup, one output per
// thread, 64 tokens per round, the next round loaded into registers while
// the current one is summed, both operands in LDS with the tokens contiguous
// (as in k_conv_valu_small).  Each output adds its tokens in ascending
// order, as k_dw_valu does, so the two give the same bits.  Measured, it is
// the faster of the two at up to 64 x 64 channels whatever the token count
// (at 32,000 tokens and 64 channels: 149 against 171 us), and otherwise while
// k_dw_valu's grid is under 256 workgroups.
constexpr int DS_M = 16, DS_N = 16, DS_K = 64, DS_P = DS_K + 4;
constexpr int DS_NMAX = 2048;                // most tokens per slice (the slice's N column sits in LDS)
constexpr int64_t kDwValuSmallBelow = 256;   // k_dw_valu workgroups under which this kernel runs
constexpr int64_t kDwValuSmallChannels = 64 * 64;   // C_in x C_out up to which it always runs

template <typename T>
__global__ __launch_bounds__(256) void k_dw_valu_small(const T* __restrict__ X, const int32_t* __restrict__ Nt,
                                                       const T* __restrict__ dY, float* __restrict__ out, int n,
                                                       int Ci, int Co, int taps, int64_t slice_tokens, int direct,
                                                       int accumulate) {
    constexpr uint32_t es = sizeof(T);
    const rsrc_t rX = make_rsrc(X, static_cast<uint32_t>(static_cast<int64_t>(n) * Ci * es));
    const rsrc_t rD = make_rsrc(dY, static_cast<uint32_t>(static_cast<int64_t>(n) * Co * es));
    __shared__ __align__(16) float sG[2][DS_M][DS_P];     // [input channel][token]
    __shared__ __align__(16) float sD[2][DS_N][DS_P];     // [output channel][token]
    __shared__ int sNc[DS_NMAX];                          // N[k][j] over the slice
    const int tilesI = (Ci + DS_M - 1) / DS_M;
    const int i0 = (blockIdx.x % tilesI) * DS_M;
    const int o0 = (blockIdx.x / tilesI) * DS_N;
    const int j = blockIdx.y;
    const int64_t kbeg = static_cast<int64_t>(blockIdx.z) * slice_tokens;
    const int64_t kend = min(static_cast<int64_t>(n), kbeg + slice_tokens);
    const int rounds = kend > kbeg ? static_cast<int>((kend - kbeg + DS_K - 1) / DS_K) : 0;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    for (int t = tid; t < kend - kbeg; t += 256) sNc[t] = clamp_index(Nt[(kbeg + t) * taps + j], n);
    __syncthreads();
    uint32_t vg[4], vd[4];
    auto fetch = [&](int r) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = tid + 256 * q;
            const int kk = e >> 4, c = e & 15;
            const int t = r * DS_K + kk;                 // token kbeg + t
            const bool in = kbeg + t < kend;
            const int m = in ? sNc[t] : -1;
            vg[q] = raw_load<T>(rX, (m >= 0 && i0 + c < Ci) ? (static_cast<uint32_t>(m) * Ci + i0 + c) * es : kOob);
            vd[q] = raw_load<T>(rD, (in && o0 + c < Co) ? (static_cast<uint32_t>(kbeg + t) * Co + o0 + c) * es
                                                        : kOob);
        }
    };
    auto commit = [&](int buf) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = tid + 256 * q;
            sG[buf][e & 15][e >> 4] = raw_f32<T>(vg[q]);
            sD[buf][e & 15][e >> 4] = raw_f32<T>(vd[q]);
        }
    };
    if (rounds > 0) {
        fetch(0);
        commit(0);
    }
    __syncthreads();
    float acc = 0.f;
    for (int r = 0; r < rounds; ++r) {
        const int cur = r & 1;
        const bool more = r + 1 < rounds;
        if (more) fetch(r + 1);
        const float* __restrict__ g = &sG[cur][ty][0];
        const float* __restrict__ d = &sD[cur][tx][0];
#pragma unroll 4
        for (int kk = 0; kk < DS_K; kk += 4)
            acc = fma4(*reinterpret_cast<const float4*>(g + kk), *reinterpret_cast<const float4*>(d + kk), acc);
        if (more) commit(cur ^ 1);
        __syncthreads();
    }
    const int i = i0 + ty, o = o0 + tx;
    if (i < Ci && o < Co) {
        float* dst = out + (direct ? static_cast<int64_t>(j) * Ci * Co
                                   : (static_cast<int64_t>(blockIdx.z) * taps + j) * Ci * Co) +
                     static_cast<int64_t>(i) * Co + o;
        *dst = (direct && accumulate) ? *dst + acc : acc;
    }
}

hipError_t launch_dw_valu(bool bf16, const void* X, const int32_t* N, const void* dY, float* out,
                          int64_t n, int Ci, int Co, int taps, int slices, int64_t slice_tokens,
                          int direct, int accumulate, hipStream_t stream) {
    const int tiles = ((Ci + VT_M - 1) / VT_M) * ((Co + VT_N - 1) / VT_N);
    dim3 grid(tiles, taps, slices);
    const int64_t es = bf16 ? 2 : 4;
    const bool small = static_cast<int64_t>(tiles) * taps * slices < kDwValuSmallBelow ||
                       static_cast<int64_t>(Ci) * Co <= kDwValuSmallChannels;
    if (small && slice_tokens <= DS_NMAX && n * Ci * es <= kMaxRange && n * Co * es <= kMaxRange) {
        const int stiles = ((Ci + DS_M - 1) / DS_M) * ((Co + DS_N - 1) / DS_N);
        const dim3 sgrid(stiles, taps, slices);
        if (bf16)
            hipLaunchKernelGGL(k_dw_valu_small<uint16_t>, sgrid, dim3(256), 0, stream,
                               static_cast<const uint16_t*>(X), N, static_cast<const uint16_t*>(dY), out,
                               static_cast<int>(n), Ci, Co, taps, slice_tokens, direct, accumulate);
        else
            hipLaunchKernelGGL(k_dw_valu_small<float>, sgrid, dim3(256), 0, stream, static_cast<const float*>(X),
                               N, static_cast<const float*>(dY), out, static_cast<int>(n), Ci, Co, taps,
                               slice_tokens, direct, accumulate);
        return hipGetLastError();
    }
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
