// bf16 gather-GEMM on the CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16,
// fp32 accumulation) for the forward pass and the input gradient.
// ("SV-TAD: Native Sparse Convolutions for Efficient Temporal Action
// Detection", Key Design 2: y_k = sum_j W_j x[N[k, j]] as an implicit GEMM
// with M = tokens, K = 9 * C_in, N = C_out; -1 entries are zero padding.)
//
// Workgroup: 256 threads = 4 waves (2 x 2); output tile 128 tokens x 128
// channels; each wave 64 x 64 = 2 x 2 blocks of 32 x 32.  Two workgroups fit
// on a compute unit (72 KiB of LDS each).
//
// Neighbour window.  Tokens are packed frame-major and, inside a frame, in
// ascending flat order, so every neighbour of token k lies within W+1 packed
// positions of k and a tile's gathered rows sit in one short range [lo, hi].
// The kernel reads the tile's N slice, finds lo/hi, and when the range holds
// at most 192 rows it stages exactly those rows (64 channels at a time, 16-byte
// coalesced loads) in LDS once for all nine taps; A fragments are then read
// from LDS by row index (N - lo; -1 maps to an all-zero row).  Tiles whose rows
// are spread wider (another packing order, grids wider than 31) fall back to
// staging the 128 gathered rows tap by tap.  Both modes feed the same MFMA
// sequence, so the result does not depend on the mode.
//
// Pipeline.  The K loop runs over rounds (64-channel chunk, tap).  At the
// start of round r the weight tile of round r + 1 goes from registers into
// the free LDS buffer and the loads of round r + 2 are issued, all ahead of
// round r's MFMAs; the next chunk's window rows load into registers half-way
// through the current chunk.  One barrier per round.  The output tile leaves
// through LDS so that global stores are whole 16-byte row pieces.
//
// Weights.  Both passes keep the weight tile in LDS as [output column][k]
// so that every MFMA fragment is one 16-byte LDS read.  Input gradient:
// B(k = o, col = i) = Wt[8-j][i][o] is already contiguous along k and is
// copied.  Forward: B(k = i, col = o) = Wt[j][i][o] is contiguous along the
// column, so half of the threads load 8 x 8 blocks and transpose them in
// registers on the way to LDS.
//
// Each round's 4 k-steps are fully unrolled with all fragment reads issued
// before the 16 MFMAs, so LDS latency overlaps the matrix work.
#include "internal.h"
#include "mfma.h"

namespace svc {

constexpr int CM_BM = 128;              // tokens per tile
constexpr int CM_BN = 128;              // output channels per tile
constexpr int CM_KC = 64;               // channels per round
constexpr int CM_WIN = 192;             // window rows held in LDS
constexpr int CM_ZROW = CM_WIN;         // an all-zero row: target of -1 entries
constexpr int CM_LDA = CM_KC + 8;       // 144 B pitch: conflict-free 16-byte row reads
constexpr int CM_LDB = CM_KC + 8;       // 144 B pitch
constexpr int CM_SB = CM_BN * CM_LDB;
constexpr int CM_WREGS = (CM_WIN * (CM_KC / 8) + 255) / 256;   // window chunks per thread (6)

// One round: KS k-steps of 16, all fragments read first, then 4 KS MFMAs.
template <int KS>
__device__ __forceinline__ void mma_round(const uint16_t* __restrict__ sA, const uint16_t* __restrict__ sb,
                                          const int arow[2], floatx16_t acc[2][2]) {
    const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 1;
    const int l32 = lane & 31, lhi = lane >> 5;
    bf16x8_t a[KS][2], b[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int kof = ks * 16 + lhi * 8;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) a[ks][mb] = frag_row(&sA[arow[mb] * CM_LDA + kof]);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) b[ks][nb] = frag_row(&sb[(wn * 64 + nb * 32 + l32) * CM_LDB + kof]);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32(a[ks][mb], b[ks][nb], acc[mb][nb]);
}

template <bool DX>
__global__ __launch_bounds__(256, 2) void k_conv_mfma(const uint16_t* __restrict__ A,
                                                      const int32_t* __restrict__ Nt,
                                                      const uint16_t* __restrict__ Wt,
                                                      const uint16_t* __restrict__ bias,
                                                      uint16_t* __restrict__ out, int n, int Ci,
                                                      int Co) {
    const int K = DX ? Co : Ci;    // contracted channels per tap
    const int NO = DX ? Ci : Co;   // produced channels

    __shared__ __align__(16) uint16_t sA[(CM_WIN + 1) * CM_LDA];
    __shared__ __align__(16) uint16_t sB[2][CM_SB];
    __shared__ int sN[CM_BM * 9];
    __shared__ short sRow[CM_BM * 9];
    __shared__ int sLo, sHi;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, lhi = lane >> 5;
    // 1-D grid: logical tile = (token tile, output-channel tile), the
    // output-channel tiles of one token range adjacent and on one XCD.
    const int tilesN = (NO + CM_BN - 1) / CM_BN;
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t k0 = static_cast<int64_t>(logical / tilesN) * CM_BM;
    const int n0 = (logical % tilesN) * CM_BN;
    const int nchunks = (K + CM_KC - 1) / CM_KC;
    const int R = nchunks * 9;

    if (tid == 0) { sLo = 0x7fffffff; sHi = -1; }
    if (tid < CM_KC / 8)
        *reinterpret_cast<uint4*>(&sA[CM_ZROW * CM_LDA + tid * 8]) = make_uint4(0, 0, 0, 0);
    __syncthreads();

    // ---- the tile's slice of N, its row range, and the LDS row of every entry
    {
        int lo = 0x7fffffff, hi = -1;
        for (int e = tid; e < CM_BM * 9; e += 256) {
            const int64_t k = k0 + e / 9;
            const int m = (k < n) ? clamp_index(Nt[k * 9 + e % 9], n) : -1;
            sN[e] = m;
            if (m >= 0) { lo = min(lo, m); hi = max(hi, m); }
        }
        if (hi >= 0) { atomicMin(&sLo, lo); atomicMax(&sHi, hi); }
    }
    __syncthreads();
    const int wlo = sLo;
    const int span = (sHi >= 0) ? sHi - wlo + 1 : 0;
    const bool window = span <= CM_WIN;
    for (int e = tid; e < CM_BM * 9; e += 256) {
        const int m = sN[e];
        sRow[e] = static_cast<short>(m < 0 ? CM_ZROW : (window ? m - wlo : e / 9));
    }

    // ---- staging helpers
    auto kc_of = [&](int c) { return min(CM_KC, K - c * CM_KC); };
    auto load_window = [&](int c, uint4* regs) {
        const int c0 = c * CM_KC, kc = kc_of(c);
#pragma unroll
        for (int u = 0; u < CM_WREGS; ++u) {
            const int q = tid + 256 * u;
            const int r = q >> 3, ch = q & 7;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (r < span && ch * 8 < kc)
                v = *reinterpret_cast<const uint4*>(A + static_cast<int64_t>(wlo + r) * K + c0 + ch * 8);
            regs[u] = v;
        }
    };
    auto store_window = [&](const uint4* regs) {
#pragma unroll
        for (int u = 0; u < CM_WREGS; ++u) {
            const int q = tid + 256 * u;
            const int r = q >> 3, ch = q & 7;
            if (r < span) *reinterpret_cast<uint4*>(&sA[r * CM_LDA + ch * 8]) = regs[u];
        }
    };
    // Weight tile of round rr (chunk rr / 9, tap rr % 9) into registers.
    // Forward: threads 0..127 each load one 8 x 8 block (8 rows k of 8
    // columns).  Input gradient: every thread loads 4 16-byte pieces.
    // Block (kb, nb) lands at LDS rows nb*8 + e, column kb*8; with the
    // 144-byte pitch its bank group is (kb + e) mod 8, so the 8 lanes that
    // share a write cycle take 8 different kb: no bank conflicts.
    auto load_B = [&](int rr, uint4* regs) {
        const int c = rr / 9, j = rr - c * 9;
        const int jt = DX ? 8 - j : j;
        const int c0 = c * CM_KC, kc = kc_of(c);
        const uint16_t* __restrict__ Wj = Wt + static_cast<int64_t>(jt) * Ci * Co;
        if (!DX) {
            if (tid < (CM_KC / 8) * (CM_BN / 8)) {
                const int kb = tid & 7, nb = tid >> 3;   // 8 neighbouring lanes: 8 k groups
                const bool ok = n0 + nb * 8 < NO;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int kk = kb * 8 + r;
                    regs[r] = (ok && kk < kc)
                                  ? *reinterpret_cast<const uint4*>(Wj + static_cast<int64_t>(c0 + kk) * Co + n0 + nb * 8)
                                  : make_uint4(0, 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int q = tid + 256 * u;
                const int nn = q >> 3, ch = q & 7;         // Wt[8-j][n0 + nn][c0 + 8 ch ...]
                uint4 v = make_uint4(0, 0, 0, 0);
                if (n0 + nn < NO && ch * 8 < kc)
                    v = *reinterpret_cast<const uint4*>(Wj + static_cast<int64_t>(n0 + nn) * Co + c0 + ch * 8);
                regs[u] = v;
            }
        }
    };
    auto store_B = [&](int buf, const uint4* regs) {
        uint16_t* sb = sB[buf];
        if (!DX) {
            if (tid < (CM_KC / 8) * (CM_BN / 8)) {
                const int kb = tid & 7, nb = tid >> 3;   // 8 neighbouring lanes: 8 k groups
                uint4 cols[8];
                transpose8x8_b16(regs, cols);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    *reinterpret_cast<uint4*>(&sb[(nb * 8 + e) * CM_LDB + kb * 8]) = cols[e];
            }
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int q = tid + 256 * u;
                const int nn = q >> 3, ch = q & 7;
                *reinterpret_cast<uint4*>(&sb[nn * CM_LDB + ch * 8]) = regs[u];
            }
        }
    };
    // Gather mode: the 128 rows of tap j, chunk c, straight into sA.
    auto stage_gather = [&](int rr) {
        const int c = rr / 9, j = rr - c * 9;
        const int c0 = c * CM_KC, kc = kc_of(c);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int q = tid + 256 * u;
            const int r = q >> 3, ch = q & 7;
            const int m = sN[r * 9 + j];
            uint4 v = make_uint4(0, 0, 0, 0);
            if (m >= 0 && ch * 8 < kc)
                v = *reinterpret_cast<const uint4*>(A + static_cast<int64_t>(m) * K + c0 + ch * 8);
            *reinterpret_cast<uint4*>(&sA[r * CM_LDA + ch * 8]) = v;
        }
    };

    floatx16_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = zero16();

    uint4 breg[8], wreg[CM_WREGS];
    if (window) {
        load_window(0, wreg);
        store_window(wreg);
    }
    load_B(0, breg);
    store_B(0, breg);
    if (R > 1) load_B(1, breg);
    __syncthreads();

    for (int r = 0; r < R; ++r) {
        const int c = r / 9, j = r - c * 9;
        if (!window) {
            stage_gather(r);
            __syncthreads();
        }
        // Stage the next round's weights into the other buffer (last read in
        // round r - 1, before the previous barrier) and start loading the
        // one after: issued ahead of this round's MFMAs so that their
        // latency hides behind the matrix work.
        if (r + 1 < R) {
            store_B((r + 1) & 1, breg);
            if (r + 2 < R) load_B(r + 2, breg);
        }
        if (window && j == 4 && c + 1 < nchunks) load_window(c + 1, wreg);
        const uint16_t* __restrict__ sb = sB[r & 1];
        int arow[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) arow[mb] = sRow[(wm * 64 + mb * 32 + l32) * 9 + j];
        // Always the full 4 k-steps: a 32-channel tail chunk is zero-filled
        // past its end in both operands, and one code path keeps the
        // accumulators in fixed registers.
        mma_round<CM_KC / 16>(sA, sb, arow, acc);
        if (r + 1 < R) {
            if (window && (r + 1) % 9 == 0) {
                __syncthreads();           // every wave is done with this chunk's window
                store_window(wreg);
            }
            __syncthreads();
        }
    }

    // ---- epilogue: bias, round to bf16, stage the 128 x 128 tile in LDS
    // (over the weight buffers), then write whole 16-byte row pieces.
    constexpr int OLD = CM_BN + 8;      // 272-byte pitch: rows 4 apart in opposite bank halves
    static_assert(CM_BM * OLD <= 2 * CM_SB, "output tile must fit the weight buffers");
    uint16_t* sOut = &sB[0][0];
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int cl = wn * 64 + nb * 32 + l32;
        const float bv = (!DX && bias && n0 + cl < NO) ? bf16_to_f32(bias[n0 + cl]) : 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    sOut[(wm * 64 + mb * 32 + g * 8 + lhi * 4 + q) * OLD + cl] = f32_to_bf16(acc[mb][nb][g * 4 + q] + bv);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < (CM_BM * CM_BN / 8) / 256; ++u) {
        const int q = tid + 256 * u;
        const int rl = q >> 4, ch = q & 15;
        const int64_t row = k0 + rl;
        const int col = n0 + ch * 8;
        if (row < n && col < NO)
            *reinterpret_cast<uint4*>(out + row * NO + col) = *reinterpret_cast<const uint4*>(&sOut[rl * OLD + ch * 8]);
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
    dim3 grid(static_cast<unsigned>(((n + CM_BM - 1) / CM_BM) * ((NO + CM_BN - 1) / CM_BN)));
    if (dx)
        hipLaunchKernelGGL(k_conv_mfma<true>, grid, dim3(256), 0, stream, A, N, Wt, bias, out,
                           static_cast<int>(n), Ci, Co);
    else
        hipLaunchKernelGGL(k_conv_mfma<false>, grid, dim3(256), 0, stream, A, N, Wt, bias, out,
                           static_cast<int>(n), Ci, Co);
    return hipGetLastError();
}

}  // namespace svc
