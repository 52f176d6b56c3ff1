// bf16 gather-GEMM on the CDNA4 matrix cores (v_mfma_f32_16x16x32_bf16,
// fp32 accumulation) for the forward pass and the input gradient.
// ("SV-TAD: Native Sparse Convolutions for Efficient Temporal Action
// Detection", Key Design 2: y_k = sum_j W_j x[N[k, j]] as an implicit GEMM
// with M = tokens, K = 9 * C_in, N = C_out; -1 entries are zero padding.)
//
// Workgroup: 256 threads = 4 waves (2 x 2), output tile 128 tokens x 128
// channels, each wave 64 x 64 = 4 x 4 MFMA blocks of 16 x 16.
//
// Neighbour window.  Tokens are packed frame-major and, inside a frame, in
// ascending flat order, so every neighbour of token k lies within W+1 packed
// positions of k.  The rows a tile gathers therefore sit in one short range
// [lo, hi] of the packed sequence.  The kernel reads the tile's N slice,
// finds lo/hi, and when hi - lo + 1 <= 256 stages exactly that contiguous
// range (64 channels at a time, fully coalesced 16-byte loads) in LDS once for
// all nine taps; the A fragments are then gathered out of LDS by row index.
// Tiles whose rows are spread wider (any other packing order) fall back to
// staging the 128 gathered rows tap by tap.  Both modes feed the same MFMA
// sequence, so results do not depend on the mode.
//
// Weights.  Forward: B(k = i, col = o) = Wt[j][i][o] is stored K-major by
// column, so each 8 x 8 block is transposed in registers on its way to LDS.
// Input gradient: B(k = o, col = i) = Wt[8-j][i][o] is already contiguous
// along K and is copied straight in.
#include "internal.h"

namespace svc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int CM_BM = 128;              // tokens per tile
constexpr int CM_BN = 128;              // output channels per tile
constexpr int CM_KC = 64;               // channels staged per round
constexpr int CM_LD = CM_KC + 8;        // LDS row pitch in bf16 (144 B: conflict-free 16 B reads)
constexpr int CM_WIN = 256;             // window rows held in LDS
constexpr int CM_ZROW = CM_WIN;         // an all-zero row: target of -1 entries

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

template <bool DX>
__global__ __launch_bounds__(256) void k_conv_mfma(const uint16_t* __restrict__ A,
                                                   const int32_t* __restrict__ Nt,
                                                   const uint16_t* __restrict__ Wt,
                                                   const uint16_t* __restrict__ bias,
                                                   uint16_t* __restrict__ out, int n, int Ci,
                                                   int Co) {
    const int K = DX ? Co : Ci;    // contracted channels per tap
    const int NO = DX ? Ci : Co;   // produced channels

    __shared__ __align__(16) uint16_t sA[(CM_WIN + 1) * CM_LD];
    __shared__ __align__(16) uint16_t sB[CM_BN * CM_LD];
    __shared__ int sN[CM_BM * 9];
    __shared__ short sRow[CM_BM * 9];
    __shared__ int sLo, sHi;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t k0 = static_cast<int64_t>(blockIdx.x) * CM_BM;
    const int n0 = blockIdx.y * CM_BN;

    if (tid == 0) { sLo = 0x7fffffff; sHi = -1; }
    for (int c = tid; c < CM_KC / 8; c += 256)
        *reinterpret_cast<uint4*>(&sA[CM_ZROW * CM_LD + c * 8]) = make_uint4(0, 0, 0, 0);
    __syncthreads();

    int lo = 0x7fffffff, hi = -1;
    for (int e = tid; e < CM_BM * 9; e += 256) {
        const int64_t k = k0 + e / 9;
        const int m = (k < n) ? clamp_index(Nt[k * 9 + e % 9], n) : -1;
        sN[e] = m;
        if (m >= 0) { lo = min(lo, m); hi = max(hi, m); }
    }
    if (hi >= 0) { atomicMin(&sLo, lo); atomicMax(&sHi, hi); }
    __syncthreads();
    const int wlo = sLo, whi = sHi;
    const int span = (whi >= 0) ? whi - wlo + 1 : 0;
    const bool window = span <= CM_WIN;
    for (int e = tid; e < CM_BM * 9; e += 256) {
        const int m = sN[e];
        sRow[e] = static_cast<short>(m < 0 ? CM_ZROW : (window ? m - wlo : e / 9));
    }

    floatx4_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    for (int c0 = 0; c0 < K; c0 += CM_KC) {
        const int kc = min(CM_KC, K - c0);   // 32 or 64 (K % 32 == 0)
        if (window) {
            __syncthreads();   // previous round's readers are done with sA
            for (int q = tid; q < span * (CM_KC / 8); q += 256) {
                const int r = q / (CM_KC / 8), ch = q % (CM_KC / 8);
                uint4 v = make_uint4(0, 0, 0, 0);
                if (ch * 8 < kc)
                    v = *reinterpret_cast<const uint4*>(A + static_cast<int64_t>(wlo + r) * K + c0 + ch * 8);
                *reinterpret_cast<uint4*>(&sA[r * CM_LD + ch * 8]) = v;
            }
        }
        for (int j = 0; j < 9; ++j) {
            const int jt = DX ? 8 - j : j;
            const uint16_t* __restrict__ Wj = Wt + static_cast<int64_t>(jt) * Ci * Co;
            __syncthreads();   // readers of sB (and of sA in gather mode) are done
            if (!window) {
                for (int q = tid; q < CM_BM * (CM_KC / 8); q += 256) {
                    const int r = q / (CM_KC / 8), ch = q % (CM_KC / 8);
                    const int m = sN[r * 9 + j];
                    uint4 v = make_uint4(0, 0, 0, 0);
                    if (m >= 0 && ch * 8 < kc)
                        v = *reinterpret_cast<const uint4*>(A + static_cast<int64_t>(m) * K + c0 + ch * 8);
                    *reinterpret_cast<uint4*>(&sA[r * CM_LD + ch * 8]) = v;
                }
            }
            if (!DX) {
                // 8 x 8 blocks of Wt[j][c0 + kk][n0 + nn], transposed into sB[nn][kk].
                if (tid < (CM_KC / 8) * (CM_BN / 8)) {
                    const int kb = tid / (CM_BN / 8), nb = tid % (CM_BN / 8);
                    uint4 rows[8], cols[8];
                    const bool col_ok = n0 + nb * 8 < NO;
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        const int kk = kb * 8 + r;
                        rows[r] = (col_ok && kk < kc)
                                      ? *reinterpret_cast<const uint4*>(Wj + static_cast<int64_t>(c0 + kk) * Co + n0 + nb * 8)
                                      : make_uint4(0, 0, 0, 0);
                    }
                    transpose8x8_b16(rows, cols);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        *reinterpret_cast<uint4*>(&sB[(nb * 8 + e) * CM_LD + kb * 8]) = cols[e];
                }
            } else {
                // sB[nn][kk] = Wt[8-j][n0 + nn][c0 + kk]: contiguous along kk.
                for (int q = tid; q < CM_BN * (CM_KC / 8); q += 256) {
                    const int nn = q / (CM_KC / 8), ch = q % (CM_KC / 8);
                    uint4 v = make_uint4(0, 0, 0, 0);
                    if (n0 + nn < NO && ch * 8 < kc)
                        v = *reinterpret_cast<const uint4*>(Wj + static_cast<int64_t>(n0 + nn) * Co + c0 + ch * 8);
                    *reinterpret_cast<uint4*>(&sB[nn * CM_LD + ch * 8]) = v;
                }
            }
            __syncthreads();

            int arow[4];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) arow[mb] = sRow[(wm * 64 + mb * 16 + (lane & 15)) * 9 + j];
            for (int ks = 0; ks < kc; ks += 32) {
                const int kof = ks + (lane >> 4) * 8;
                bf16x8_t a[4], b[4];
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
                    a[mb] = as_bf16x8(*reinterpret_cast<const uint4*>(&sA[arow[mb] * CM_LD + kof]));
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    b[nb] = as_bf16x8(*reinterpret_cast<const uint4*>(
                        &sB[(wn * 64 + nb * 16 + (lane & 15)) * CM_LD + kof]));
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb)
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb], b[nb], acc[mb][nb], 0, 0, 0);
            }
        }
    }

    // D fragment: lane holds rows 4*(lane/16) .. +3 of column lane%16.
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const int col = n0 + wn * 64 + nb * 16 + (lane & 15);
        if (col >= NO) continue;
        const float bv = (!DX && bias) ? bf16_to_f32(bias[col]) : 0.f;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t row = k0 + wm * 64 + mb * 16 + (lane >> 4) * 4 + q;
                if (row < n) out[row * NO + col] = f32_to_bf16(acc[mb][nb][q] + bv);
            }
        }
    }
}

bool conv_mfma_supported(bool dx, int Ci, int Co) {
    const int K = dx ? Co : Ci, NO = dx ? Ci : Co;
    return K > 0 && NO > 0 && K % 32 == 0 && NO % 16 == 0;
}

hipError_t launch_conv_mfma(bool dx, const uint16_t* A, const int32_t* N, const uint16_t* Wt,
                            const uint16_t* bias, uint16_t* out, int64_t n, int Ci, int Co,
                            hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int NO = dx ? Ci : Co;
    dim3 grid(static_cast<unsigned>((n + CM_BM - 1) / CM_BM), static_cast<unsigned>((NO + CM_BN - 1) / CM_BN));
    if (dx)
        hipLaunchKernelGGL(k_conv_mfma<true>, grid, dim3(256), 0, stream, A, N, Wt, bias, out,
                           static_cast<int>(n), Ci, Co);
    else
        hipLaunchKernelGGL(k_conv_mfma<false>, grid, dim3(256), 0, stream, A, N, Wt, bias, out,
                           static_cast<int>(n), Ci, Co);
    return hipGetLastError();
}

}  // namespace svc
