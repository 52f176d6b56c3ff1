// Asymmetric cross-attention ("SV-TAD: Native Sparse Convolutions for
// Efficient Temporal Action Detection", Key Design 3): a few auxiliary
// tokens Q [m][d] query the down-projected sparse visual tokens X [n][d],
// which are both keys and values, and only the auxiliary tokens are updated:
//   S[q][j] = scale <Q[q], X[j]>,  P = row softmax of S,  O = P X.
// Single head, no further projections (the page prints no more than that).
//
// The work is a read of X (n d elements) against a handful of queries, so it
// is bound by HBM bandwidth, and it is split over key blocks like a split-K
// reduction:
//   forward:  each workgroup folds its key block into a running maximum,
//             sum and weighted row sum per query (the online softmax) and
//             writes them as a partial; a second kernel merges the partials
//             in block order into O and lse = log sum_j exp S[q][j].
//   backward: with lse from the forward, P is recomputed per key; a first
//             pass sums D[q] = sum_j P[q][j] <dO[q], X[j]> per key block (keys
//             shifted by O[q], see the backward section), a second writes each
//             key's row of
//               dX[j] = scale sum_q dS[q][j] Q[q] + sum_q P[q][j] dO[q],
//               dS[q][j] = P[q][j] (<dO[q], X[j]> - D[q]),
//             and block partials of dQ[q] = scale sum_j dS[q][j] X[j], merged
//             in block order.
// Everything is summed in a fixed order, so results are bitwise
// reproducible.
//
// Lanes: 16 lanes share a key row, each holding d / 16 consecutive elements
// (one or two 16-byte loads), so a row is one contiguous 2d- or 4d-byte read;
// a workgroup of 256 threads has 16 such groups.  Dot products finish with
// four butterfly exchanges inside the 16-lane group.  Queries go through in
// chunks held in registers (one query, the CLS case, has its own
// instantiation).
#include "internal.h"

namespace svc {

// 64-bit minimum (the unqualified device min() may resolve to its int
// overload and truncate).
__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }


constexpr int XA_THREADS = 256;
constexpr int XA_GROUPS = XA_THREADS / 16;
constexpr int XA_MQ = 4;                 // queries per pass

template <typename T, int EPL>
__device__ __forceinline__ void load_part(const T* __restrict__ p, float (&v)[EPL]) {
    if constexpr (sizeof(T) == 2) {
        static_assert(EPL % 4 == 0, "bf16 pieces of 8 bytes at least");
        if constexpr (EPL % 8 == 0) {
#pragma unroll
            for (int u = 0; u < EPL / 8; ++u) {
                const uint4 w = reinterpret_cast<const uint4*>(p)[u];
                const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    v[8 * u + 2 * h] = __uint_as_float(a[h] << 16);
                    v[8 * u + 2 * h + 1] = __uint_as_float(a[h] & 0xffff0000u);
                }
            }
        } else {
            const uint2 w = *reinterpret_cast<const uint2*>(p);
            v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xffff0000u);
            v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int u = 0; u < EPL / 4; ++u) {
            const float4 w = reinterpret_cast<const float4*>(p)[u];
            v[4 * u] = w.x; v[4 * u + 1] = w.y; v[4 * u + 2] = w.z; v[4 * u + 3] = w.w;
        }
    }
}

template <typename T, int EPL>
__device__ __forceinline__ void store_part(T* __restrict__ p, const float (&v)[EPL]) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < EPL; e += 4) {
            const uint32_t lo = f32_to_bf16(v[e]) | (static_cast<uint32_t>(f32_to_bf16(v[e + 1])) << 16);
            const uint32_t hi = f32_to_bf16(v[e + 2]) | (static_cast<uint32_t>(f32_to_bf16(v[e + 3])) << 16);
            *reinterpret_cast<uint2*>(p + e) = make_uint2(lo, hi);
        }
    } else {
#pragma unroll
        for (int e = 0; e < EPL; e += 4) *reinterpret_cast<float4*>(p + e) = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
    }
}

// Sum over the 16 lanes of a group; every lane receives the total.
__device__ __forceinline__ float group_sum(float s) {
#pragma unroll
    for (int k = 8; k >= 1; k >>= 1) s += __shfl_xor(s, k, 16);
    return s;
}

// ---------------------------------------------------------------- forward
// Partials per (key block b, query q): pM[b][q] (largest score), pL[b][q]
// (sum of exp(S - pM)) and pA[b][q][:] (sum of exp(S - pM) X[j]).  A block
// without keys writes pM = -inf, pL = 0, pA = 0.
template <typename T, int EPL, int MQ>
__global__ __launch_bounds__(XA_THREADS) void k_xattn_fwd_part(const T* __restrict__ Q, const T* __restrict__ X,
                                                               int m, int64_t n, float scale, int64_t kpb,
                                                               float* __restrict__ pM, float* __restrict__ pL,
                                                               float* __restrict__ pA) {
    constexpr int D = 16 * EPL;
    constexpr int WAVES = XA_THREADS / 64;
    __shared__ float sM[WAVES][MQ], sL[WAVES][MQ];
    __shared__ float sA[WAVES][MQ][D];
    const int tid = threadIdx.x, lane = tid & 15, grp = tid >> 4, wave = tid >> 6;
    const int64_t b = blockIdx.x;
    const int q0 = blockIdx.y * MQ, mq = min(MQ, m - q0);

    float qv[MQ][EPL], acc[MQ][EPL], M[MQ], L[MQ];
#pragma unroll
    for (int qi = 0; qi < MQ; ++qi) {
        if (qi < mq) load_part<T, EPL>(Q + static_cast<int64_t>(q0 + qi) * D + lane * EPL, qv[qi]);
        else
#pragma unroll
            for (int e = 0; e < EPL; ++e) qv[qi][e] = 0.f;
        M[qi] = -INFINITY;
        L[qi] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[qi][e] = 0.f;
    }
    // Each group walks its keys two at a time with the next two rows already
    // requested (request indices are clamped into the block, so no load sits
    // behind a branch).
    const int64_t kbeg = b * kpb, kend = min64(n, kbeg + kpb);
    auto row = [&](int64_t j) { return X + min64(j, kend - 1) * D + lane * EPL; };
    auto fold = [&](const float* x) {
#pragma unroll
        for (int qi = 0; qi < MQ; ++qi) {
            if (qi >= mq) break;
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) s = fmaf(x[e], qv[qi][e], s);
            s = scale * group_sum(s);
            const float mn = fmaxf(M[qi], s);
            const float corr = __expf(M[qi] - mn);        // 0 on the first key (M = -inf)
            const float p = __expf(s - mn);
            L[qi] = fmaf(L[qi], corr, p);
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[qi][e] = fmaf(acc[qi][e], corr, p * x[e]);
            M[qi] = mn;
        }
    };
    float x0[EPL], x1[EPL];
    load_part<T, EPL>(row(kbeg + grp), x0);
    load_part<T, EPL>(row(kbeg + grp + XA_GROUPS), x1);
    for (int64_t j = kbeg + grp; j < kend; j += 2 * XA_GROUPS) {
        float n0[EPL], n1[EPL];
        load_part<T, EPL>(row(j + 2 * XA_GROUPS), n0);
        load_part<T, EPL>(row(j + 3 * XA_GROUPS), n1);
        fold(x0);
        if (j + XA_GROUPS < kend) fold(x1);
#pragma unroll
        for (int e = 0; e < EPL; ++e) { x0[e] = n0[e]; x1[e] = n1[e]; }
    }
    // Merge the four groups of a wave (pairs 16 lanes apart, then 32: the
    // same dims of another group; both partners compute the same sums), then
    // the four waves in wave order.
#pragma unroll
    for (int qi = 0; qi < MQ; ++qi)
#pragma unroll
        for (int k = 16; k <= 32; k <<= 1) {
            const float om = __shfl_xor(M[qi], k, 64), ol = __shfl_xor(L[qi], k, 64);
            const float mx = fmaxf(M[qi], om);
            const float w0 = M[qi] == -INFINITY ? 0.f : __expf(M[qi] - mx);
            const float w1 = om == -INFINITY ? 0.f : __expf(om - mx);
            L[qi] = L[qi] * w0 + ol * w1;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[qi][e] = acc[qi][e] * w0 + __shfl_xor(acc[qi][e], k, 64) * w1;
            M[qi] = mx;
        }
    if ((tid & 63) < 16)
#pragma unroll
        for (int qi = 0; qi < MQ; ++qi) {
            if (lane == 0) { sM[wave][qi] = M[qi]; sL[wave][qi] = L[qi]; }
#pragma unroll
            for (int e = 0; e < EPL; ++e) sA[wave][qi][lane * EPL + e] = acc[qi][e];
        }
    __syncthreads();
    for (int t = tid; t < mq * D; t += XA_THREADS) {
        const int qi = t / D, c = t - qi * D;
        float mx = -INFINITY;
        for (int g = 0; g < WAVES; ++g) mx = fmaxf(mx, sM[g][qi]);
        float l = 0.f, a = 0.f;
        if (mx != -INFINITY)
            for (int g = 0; g < WAVES; ++g) {
                const float w = sM[g][qi] == -INFINITY ? 0.f : __expf(sM[g][qi] - mx);
                l = fmaf(sL[g][qi], w, l);
                a = fmaf(sA[g][qi][c], w, a);
            }
        const int64_t o = b * m + q0 + qi;
        pA[o * D + c] = a;
        if (c == 0) { pM[o] = mx; pL[o] = l; }
    }
}

// Merge of the block partials.  Workgroup = (query q, 16 columns); thread
// (column tid % 16, slice tid / 16) sums the blocks b = slice (mod 16) in
// ascending order, eight requests in flight, and the 16 slice sums are added
// in slice order.  The forward weights w_b = exp(pM[b][q] - max_b pM[b][q])
// are computed once per workgroup into LDS.  XA_MAX_BLOCKS bounds B (the
// plan stays below it).
constexpr int XA_MAX_BLOCKS = 2048;
constexpr int XA_MCOLS = 16;

__device__ __forceinline__ float slice_sum(const float* __restrict__ part, const float* __restrict__ w, int64_t blocks,
                                           int64_t stride, int slice) {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int64_t b = slice;
    for (; b + 7 * 16 < blocks; b += 8 * 16) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = part[(b + 16 * u) * stride];
#pragma unroll
        for (int u = 0; u < 8; ++u) a[u] = fmaf(v[u], w ? w[b + 16 * u] : 1.f, a[u]);
    }
    for (int u = 0; b < blocks; b += 16, ++u) a[u & 7] = fmaf(part[b * stride], w ? w[b] : 1.f, a[u & 7]);
    return ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
}

__device__ __forceinline__ float slices_total(float v, float (*red)[XA_MCOLS]) {
    const int c = threadIdx.x % XA_MCOLS, slice = threadIdx.x / XA_MCOLS;
    red[slice][c] = v;
    __syncthreads();
    float t = 0.f;
    for (int k = 0; k < XA_THREADS / XA_MCOLS; ++k) t += red[k][c];
    return t;
}

template <typename T>
__global__ __launch_bounds__(XA_THREADS) void k_xattn_fwd_merge(const float* __restrict__ pM, const float* __restrict__ pL,
                                                                const float* __restrict__ pA, int64_t blocks, int m,
                                                                int d, T* __restrict__ O, float* __restrict__ lse) {
    __shared__ float sW[XA_MAX_BLOCKS];
    __shared__ float sRed[XA_THREADS / XA_MCOLS][XA_MCOLS];
    __shared__ float sMax[XA_THREADS / 64], sSum[XA_THREADS / 64];
    const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float mx = -INFINITY;
    for (int64_t b = tid; b < blocks; b += XA_THREADS) mx = fmaxf(mx, pM[b * m + q]);
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) mx = fmaxf(mx, __shfl_xor(mx, k, 64));
    if (lane == 0) sMax[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(sMax[0], sMax[1]), fmaxf(sMax[2], sMax[3]));
    // weights, and the weighted count l = sum_b pL[b][q] w_b (thread sums in
    // block order, then a fixed tree)
    float l = 0.f;
    for (int64_t b = tid; b < blocks; b += XA_THREADS) {
        const float pm = pM[b * m + q];
        const float wb = (mx == -INFINITY || pm == -INFINITY) ? 0.f : __expf(pm - mx);
        sW[b] = wb;
        l = fmaf(pL[b * m + q], wb, l);
    }
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) l += __shfl_xor(l, k, 64);
    if (lane == 0) sSum[wave] = l;
    __syncthreads();
    l = (sSum[0] + sSum[1]) + (sSum[2] + sSum[3]);
    const int c = blockIdx.y * XA_MCOLS + tid % XA_MCOLS;
    const float v = c < d ? slice_sum(pA + static_cast<int64_t>(q) * d + c, sW, blocks,
                                      static_cast<int64_t>(m) * d, tid / XA_MCOLS) : 0.f;
    const float a = slices_total(v, sRed);
    if (tid < XA_MCOLS && c < d) Elem<T>::store(O + static_cast<int64_t>(q) * d + c, l > 0.f ? a / l : 0.f);
    if (blockIdx.y == 0 && tid == 0) lse[q] = (mx == -INFINITY || !(l > 0.f)) ? -INFINITY : mx + __logf(l);
}

// --------------------------------------------------------------- backward
// Conditioning.  dS[q][j] = P (dP[q][j] - D[q]) sums to zero over j, so dQ
// and dS do not change when every key row is shifted by the same vector c
// (the scores shift by a constant per query, which the softmax ignores).
// When the tokens share a large component, the unshifted sums
// sum_j dS X[j] and the dot products dP cancel to a small remainder and
// fp32 loses it; with c = O[q] (the forward output, the softmax-weighted
// mean of the keys) the shifted rows X[j] - O[q] are small and the sums are
// well conditioned.  O only serves as this shift: any vector gives the same
// result in exact arithmetic.
//   dP~[q][j] = <dO[q], X[j] - O[q]>,  D~[q] = sum_j P dP~  (pass 1, block
//   sums pS[b][q] added in block order by pass 2),  dS = P (dP~ - D~),
//   dQ[q] = scale sum_j dS (X[j] - O[q]).
//
// Pass 1, queries q0 .. q0 + MQ - 1.
template <typename T, int EPL, int MQ>
__global__ __launch_bounds__(XA_THREADS) void k_xattn_bwd_dsum(const T* __restrict__ Q, const T* __restrict__ X,
                                                               const T* __restrict__ O, const T* __restrict__ dO,
                                                               const float* __restrict__ lse, int m, int q0, int64_t n,
                                                               float scale, int64_t kpb, float* __restrict__ pS) {
    constexpr int D = 16 * EPL;
    constexpr int WAVES = XA_THREADS / 64;
    __shared__ float sS[WAVES][MQ];
    const int tid = threadIdx.x, lane = tid & 15, grp = tid >> 4, wave = tid >> 6;
    const int64_t b = blockIdx.x;
    const int mq = min(MQ, m - q0);
    float qv[MQ][EPL], gv[MQ][EPL], cv[MQ][EPL], lq[MQ], ss[MQ];
#pragma unroll
    for (int qi = 0; qi < MQ; ++qi) {
        if (qi < mq) {
            load_part<T, EPL>(Q + static_cast<int64_t>(q0 + qi) * D + lane * EPL, qv[qi]);
            load_part<T, EPL>(dO + static_cast<int64_t>(q0 + qi) * D + lane * EPL, gv[qi]);
            load_part<T, EPL>(O + static_cast<int64_t>(q0 + qi) * D + lane * EPL, cv[qi]);
            lq[qi] = lse[q0 + qi];
        } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) { qv[qi][e] = 0.f; gv[qi][e] = 0.f; cv[qi][e] = 0.f; }
            lq[qi] = 0.f;
        }
        ss[qi] = 0.f;
    }
    const int64_t kbeg = b * kpb, kend = min64(n, kbeg + kpb);
    auto row = [&](int64_t j) { return X + min64(j, kend - 1) * D + lane * EPL; };
    auto fold = [&](const float* x) {
#pragma unroll
        for (int qi = 0; qi < MQ; ++qi) {
            if (qi >= mq) break;
            float s = 0.f, g = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                s = fmaf(x[e], qv[qi][e], s);
                g = fmaf(x[e] - cv[qi][e], gv[qi][e], g);
            }
            s = group_sum(s);
            g = group_sum(g);
            ss[qi] = fmaf(__expf(scale * s - lq[qi]), g, ss[qi]);
        }
    };
    float x0[EPL], x1[EPL];
    load_part<T, EPL>(row(kbeg + grp), x0);
    load_part<T, EPL>(row(kbeg + grp + XA_GROUPS), x1);
    for (int64_t j = kbeg + grp; j < kend; j += 2 * XA_GROUPS) {
        float n0[EPL], n1[EPL];
        load_part<T, EPL>(row(j + 2 * XA_GROUPS), n0);
        load_part<T, EPL>(row(j + 3 * XA_GROUPS), n1);
        fold(x0);
        if (j + XA_GROUPS < kend) fold(x1);
#pragma unroll
        for (int e = 0; e < EPL; ++e) { x0[e] = n0[e]; x1[e] = n1[e]; }
    }
#pragma unroll
    for (int qi = 0; qi < MQ; ++qi) {
        ss[qi] += __shfl_xor(ss[qi], 16, 64);
        ss[qi] += __shfl_xor(ss[qi], 32, 64);
    }
    if ((tid & 63) == 0)
#pragma unroll
        for (int qi = 0; qi < MQ; ++qi) sS[wave][qi] = ss[qi];
    __syncthreads();
    if (tid < mq) pS[b * m + q0 + tid] = ((sS[0][tid] + sS[1][tid]) + sS[2][tid]) + sS[3][tid];
}

// Pass 2, the same queries: D[q] from the block sums (in block order, then a
// fixed tree), dS = P (dP - D) per key; dX rows are written (accumulate = 0)
// or added to (later query chunks); dQ block partials go to pQ[b][q][:].
template <typename T, int EPL, int MQ>
__global__ __launch_bounds__(XA_THREADS) void k_xattn_bwd_part(const T* __restrict__ Q, const T* __restrict__ X,
                                                               const T* __restrict__ O, const T* __restrict__ dO,
                                                               const float* __restrict__ lse,
                                                               const float* __restrict__ pS, int64_t blocks, int m,
                                                               int q0, int64_t n, float scale, int64_t kpb,
                                                               int accumulate, T* __restrict__ dX,
                                                               float* __restrict__ pQ) {
    constexpr int D = 16 * EPL;
    constexpr int WAVES = XA_THREADS / 64;
    __shared__ float sD[WAVES][MQ];
    __shared__ float sQ[WAVES][MQ][D];
    const int tid = threadIdx.x, lane = tid & 15, grp = tid >> 4, wave = tid >> 6;
    const int64_t b = blockIdx.x;
    const int mq = min(MQ, m - q0);

    float Dq[MQ];
#pragma unroll
    for (int qi = 0; qi < MQ; ++qi) {
        float v = 0.f;
        if (qi < mq)
            for (int64_t bb = tid; bb < blocks; bb += XA_THREADS) v += pS[bb * m + q0 + qi];
#pragma unroll
        for (int k = 32; k >= 1; k >>= 1) v += __shfl_xor(v, k, 64);
        if ((tid & 63) == 0) sD[wave][qi] = v;
    }
    __syncthreads();
#pragma unroll
    for (int qi = 0; qi < MQ; ++qi) Dq[qi] = (sD[0][qi] + sD[1][qi]) + (sD[2][qi] + sD[3][qi]);

    float qv[MQ][EPL], gv[MQ][EPL], cv[MQ][EPL], dq[MQ][EPL], lq[MQ];
#pragma unroll
    for (int qi = 0; qi < MQ; ++qi) {
        if (qi < mq) {
            load_part<T, EPL>(Q + static_cast<int64_t>(q0 + qi) * D + lane * EPL, qv[qi]);
            load_part<T, EPL>(dO + static_cast<int64_t>(q0 + qi) * D + lane * EPL, gv[qi]);
            load_part<T, EPL>(O + static_cast<int64_t>(q0 + qi) * D + lane * EPL, cv[qi]);
            lq[qi] = lse[q0 + qi];
        } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) { qv[qi][e] = 0.f; gv[qi][e] = 0.f; cv[qi][e] = 0.f; }
            lq[qi] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) dq[qi][e] = 0.f;
    }

    const int64_t kbeg = b * kpb, kend = min64(n, kbeg + kpb);
    auto row = [&](int64_t j) { return X + min64(j, kend - 1) * D + lane * EPL; };
    auto key = [&](int64_t j, const float* x) {
        float dx[EPL];
        if (accumulate) load_part<T, EPL>(dX + j * D + lane * EPL, dx);
        else
#pragma unroll
            for (int e = 0; e < EPL; ++e) dx[e] = 0.f;
#pragma unroll
        for (int qi = 0; qi < MQ; ++qi) {
            if (qi >= mq) break;
            float s = 0.f, g = 0.f, xc[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                xc[e] = x[e] - cv[qi][e];
                s = fmaf(x[e], qv[qi][e], s);
                g = fmaf(xc[e], gv[qi][e], g);
            }
            s = group_sum(s);
            g = group_sum(g);
            const float p = __expf(scale * s - lq[qi]);
            const float ks = scale * p * (g - Dq[qi]);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                dx[e] = fmaf(ks, qv[qi][e], fmaf(p, gv[qi][e], dx[e]));
                dq[qi][e] = fmaf(ks, xc[e], dq[qi][e]);
            }
        }
        store_part<T, EPL>(dX + j * D + lane * EPL, dx);
    };
    float x0[EPL], x1[EPL];
    load_part<T, EPL>(row(kbeg + grp), x0);
    load_part<T, EPL>(row(kbeg + grp + XA_GROUPS), x1);
    for (int64_t j = kbeg + grp; j < kend; j += 2 * XA_GROUPS) {
        float n0[EPL], n1[EPL];
        load_part<T, EPL>(row(j + 2 * XA_GROUPS), n0);
        load_part<T, EPL>(row(j + 3 * XA_GROUPS), n1);
        key(j, x0);
        if (j + XA_GROUPS < kend) key(j + XA_GROUPS, x1);
#pragma unroll
        for (int e = 0; e < EPL; ++e) { x0[e] = n0[e]; x1[e] = n1[e]; }
    }
    // dQ partial of the block: the groups of a wave added pairwise (16 lanes
    // apart, then 32), then the waves in wave order.
#pragma unroll
    for (int qi = 0; qi < MQ; ++qi)
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            dq[qi][e] += __shfl_xor(dq[qi][e], 16, 64);
            dq[qi][e] += __shfl_xor(dq[qi][e], 32, 64);
        }
    if ((tid & 63) < 16)
#pragma unroll
        for (int qi = 0; qi < MQ; ++qi)
#pragma unroll
            for (int e = 0; e < EPL; ++e) sQ[wave][qi][lane * EPL + e] = dq[qi][e];
    __syncthreads();
    for (int t = tid; t < mq * D; t += XA_THREADS) {
        const int qi = t / D, c = t - qi * D;
        float a = 0.f;
        for (int g = 0; g < WAVES; ++g) a += sQ[g][qi][c];
        pQ[(b * m + q0 + qi) * D + c] = a;
    }
}

// dQ[q][c] = sum_b pQ[b][q][c]; same layout as the forward merge.
__global__ __launch_bounds__(XA_THREADS) void k_xattn_dq_merge(const float* __restrict__ pQ, int64_t blocks, int m,
                                                               int d, float* __restrict__ dQ) {
    __shared__ float sRed[XA_THREADS / XA_MCOLS][XA_MCOLS];
    const int q = blockIdx.x, tid = threadIdx.x;
    const int c = blockIdx.y * XA_MCOLS + tid % XA_MCOLS;
    const int64_t off = static_cast<int64_t>(q) * d + c;
    const float v = c < d ? slice_sum(pQ + off, nullptr, blocks, static_cast<int64_t>(m) * d, tid / XA_MCOLS) : 0.f;
    const float a = slices_total(v, sRed);
    if (tid < XA_MCOLS && c < d) dQ[off] = a;
}

// ------------------------------------------------------------------- host
// Keys per block: about 512 blocks over n (never more than XA_MAX_BLOCKS),
// a multiple of the 16 groups.
XattnPlan plan_xattn(int64_t m, int64_t n, int d) {
    XattnPlan p{};
    p.kpb = std::max<int64_t>(XA_GROUPS, ((n + 511) / 512 + XA_GROUPS - 1) / XA_GROUPS * XA_GROUPS);
    p.blocks = n > 0 ? (n + p.kpb - 1) / p.kpb : 0;
    auto up = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
    const size_t mb = static_cast<size_t>(m) * p.blocks;
    p.fwd_bytes = up(mb * 4) * 2 + up(mb * d * 4);
    p.bwd_bytes = up(mb * d * 4) + up(mb * 4);
    return p;
}

bool xattn_supported(int d) { return d == 64 || d == 128 || d == 256; }

template <typename T, int EPL>
static hipError_t fwd_as(const XattnPlan& p, const T* Q, const T* X, int m, int64_t n, float scale, T* O,
                         float* lse, void* ws, hipStream_t stream) {
    auto up = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
    const size_t mb = static_cast<size_t>(m) * p.blocks;
    float* pM = static_cast<float*>(ws);
    float* pL = reinterpret_cast<float*>(static_cast<char*>(ws) + up(mb * 4));
    float* pA = reinterpret_cast<float*>(static_cast<char*>(ws) + 2 * up(mb * 4));
    if (p.blocks > 0) {
        // one query (the CLS token) gets an instantiation with a quarter of
        // the registers, hence twice the waves per SIMD
        if (m == 1)
            hipLaunchKernelGGL((k_xattn_fwd_part<T, EPL, 1>), dim3(static_cast<unsigned>(p.blocks)), dim3(XA_THREADS),
                               0, stream, Q, X, m, n, scale, p.kpb, pM, pL, pA);
        else
            hipLaunchKernelGGL((k_xattn_fwd_part<T, EPL, XA_MQ>),
                               dim3(static_cast<unsigned>(p.blocks), static_cast<unsigned>((m + XA_MQ - 1) / XA_MQ)),
                               dim3(XA_THREADS), 0, stream, Q, X, m, n, scale, p.kpb, pM, pL, pA);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_xattn_fwd_merge<T>, dim3(m, 16 * EPL / XA_MCOLS), dim3(XA_THREADS), 0, stream, pM, pL, pA,
                       p.blocks, m, 16 * EPL, O, lse);
    return hipGetLastError();
}

template <typename T, int EPL>
static hipError_t bwd_as(const XattnPlan& p, const T* Q, const T* X, const T* O, const T* dO, const float* lse, int m,
                         int64_t n, float scale, float* dQ, T* dX, void* ws, hipStream_t stream) {
    constexpr int MQ = EPL >= 16 ? 2 : 4;
    auto up = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
    const size_t mb = static_cast<size_t>(m) * p.blocks;
    float* pQ = static_cast<float*>(ws);
    float* pS = reinterpret_cast<float*>(static_cast<char*>(ws) + up(mb * 16 * EPL * 4));
    const dim3 grid(static_cast<unsigned>(p.blocks));
    hipError_t e = hipSuccess;
    if (p.blocks > 0 && m == 1) {
        hipLaunchKernelGGL((k_xattn_bwd_dsum<T, EPL, 1>), grid, dim3(XA_THREADS), 0, stream, Q, X, O, dO, lse, m, 0,
                           n, scale, p.kpb, pS);
        hipLaunchKernelGGL((k_xattn_bwd_part<T, EPL, 1>), grid, dim3(XA_THREADS), 0, stream, Q, X, O, dO, lse, pS,
                           p.blocks, m, 0, n, scale, p.kpb, 0, dX, pQ);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if (p.blocks > 0) {
        for (int q0 = 0; q0 < m; q0 += MQ) {
            hipLaunchKernelGGL((k_xattn_bwd_dsum<T, EPL, MQ>), grid, dim3(XA_THREADS), 0, stream, Q, X, O, dO, lse, m,
                               q0, n, scale, p.kpb, pS);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        for (int q0 = 0; q0 < m; q0 += MQ) {
            hipLaunchKernelGGL((k_xattn_bwd_part<T, EPL, MQ>), grid, dim3(XA_THREADS), 0, stream, Q, X, O, dO, lse,
                               pS, p.blocks, m, q0, n, scale, p.kpb, q0 > 0 ? 1 : 0, dX, pQ);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    hipLaunchKernelGGL(k_xattn_dq_merge, dim3(m, 16 * EPL / XA_MCOLS), dim3(XA_THREADS), 0, stream, pQ, p.blocks, m,
                       16 * EPL, dQ);
    return hipGetLastError();
}

hipError_t launch_xattn_fwd(const XattnPlan& p, bool bf16, const void* Q, const void* X, int m, int64_t n, int d,
                            float scale, void* O, float* lse, void* ws, hipStream_t stream) {
#define XA_FWD(T, EPL)                                                                                         \
    return fwd_as<T, EPL>(p, static_cast<const T*>(Q), static_cast<const T*>(X), m, n, scale, static_cast<T*>(O), \
                          lse, ws, stream)
    if (bf16) {
        if (d == 64) XA_FWD(uint16_t, 4);
        if (d == 128) XA_FWD(uint16_t, 8);
        XA_FWD(uint16_t, 16);
    }
    if (d == 64) XA_FWD(float, 4);
    if (d == 128) XA_FWD(float, 8);
    XA_FWD(float, 16);
#undef XA_FWD
}

hipError_t launch_xattn_bwd(const XattnPlan& p, bool bf16, const void* Q, const void* X, const void* O,
                            const void* dO, const float* lse, int m, int64_t n, int d, float scale, float* dQ,
                            void* dX, void* ws, hipStream_t stream) {
#define XA_BWD(T, EPL)                                                                                         \
    return bwd_as<T, EPL>(p, static_cast<const T*>(Q), static_cast<const T*>(X), static_cast<const T*>(O),     \
                          static_cast<const T*>(dO), lse, m, n, scale, dQ, static_cast<T*>(dX), ws, stream)
    if (bf16) {
        if (d == 64) XA_BWD(uint16_t, 4);
        if (d == 128) XA_BWD(uint16_t, 8);
        XA_BWD(uint16_t, 16);
    }
    if (d == 64) XA_BWD(float, 4);
    if (d == 128) XA_BWD(float, 8);
    XA_BWD(float, 16);
#undef XA_BWD
}

}  // namespace svc
