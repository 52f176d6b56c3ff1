// Neighbour index table on the GPU ("SV-TAD: Native Sparse Convolutions for
// Efficient Temporal Action Detection", Key Design 1: the lookup map M and
// the neighbour table N, both O(N_kept)).
//
// One workgroup per frame.  The frame's map lives in LDS (H*W int32, at most
// 64 KiB): fill with -1, scatter M[p_k] = k with an atomic exchange (a
// previous value other than -1 means two tokens on one cell), then each
// thread produces consecutive elements of the frame's contiguous N block, so
// the rows (K*K int32 each) are written fully coalesced.  The neighbourhood
// is K x K (K odd), tap j = K (dy + K/2) + (dx + K/2) for offsets dy, dx in
// [-K/2, K/2]: the 3 x 3 case is the one the page builds.
#include "internal.h"

namespace svc {

constexpr int kIndexThreads = 256;

__global__ __launch_bounds__(kIndexThreads) void k_build_index(
    const int32_t* __restrict__ coords, const int32_t* __restrict__ offs, int frame_begin,
    int H, int W, int K, int64_t n_rows, int64_t tok_base, int32_t* __restrict__ N,
    int32_t* __restrict__ M, int32_t* __restrict__ err) {
    extern __shared__ int32_t smap[];
    const int cells = H * W;
    const int t = frame_begin + static_cast<int>(blockIdx.x);
    const int64_t beg = offs[t], end = offs[t + 1];
    int flag = 0;
    // The frame's rows must lie inside the caller's N buffer.
    const bool ok = beg >= tok_base && end >= beg && end - tok_base <= n_rows &&
                    end - beg <= cells;
    if (!ok) flag |= SV_FLAG_BAD_OFFSETS;

    for (int c = threadIdx.x; c < cells; c += kIndexThreads) smap[c] = -1;
    __syncthreads();

    // Step 1: M[p_k] = k (indices relative to tok_base).
    if (ok) {
        for (int64_t k = beg + threadIdx.x; k < end; k += kIndexThreads) {
            const int p = coords[k];
            if (static_cast<unsigned>(p) >= static_cast<unsigned>(cells)) {
                flag |= SV_FLAG_COORD_RANGE;
                continue;
            }
            const int old = atomicExch(&smap[p], static_cast<int>(k - tok_base));
            if (old != -1) flag |= SV_FLAG_DUPLICATE;
        }
    }
    __syncthreads();

    // Step 2: N[k][j] = M[y + dy_j][x + dx_j], bounds checked per axis.
    if (ok) {
        const int taps = K * K, rad = K / 2;
        const int total = static_cast<int>(end - beg) * taps;   // <= 16384 * 49
        int32_t* __restrict__ Nf = N + (beg - tok_base) * taps;
        const int32_t* __restrict__ cf = coords + beg;
        for (int e = threadIdx.x; e < total; e += kIndexThreads) {
            const int r = e / taps;
            const int j = e - r * taps;
            const int p = cf[r];
            int v = -1;
            if (static_cast<unsigned>(p) < static_cast<unsigned>(cells)) {
                const int y = p / W, x = p - y * W;
                const int dy = j / K;
                const int yy = y + dy - rad, xx = x + (j - dy * K) - rad;
                if (yy >= 0 && yy < H && xx >= 0 && xx < W) v = smap[yy * W + xx];
            }
            Nf[e] = v;
        }
    }
    if (M) {
        int32_t* Mf = M + static_cast<int64_t>(blockIdx.x) * cells;
        for (int c = threadIdx.x; c < cells; c += kIndexThreads) Mf[c] = smap[c];
    }
    if (flag && err) atomicOr(err, flag);
}

hipError_t launch_build_index(const int32_t* coords, const int32_t* offs, int frame_begin,
                              int frames, int H, int W, int K, int64_t n_rows, int64_t tok_base,
                              int32_t* N, int32_t* M, int32_t* err, hipStream_t stream) {
    if (frames <= 0) return hipSuccess;
    const size_t lds = sizeof(int32_t) * static_cast<size_t>(H) * W;
    hipLaunchKernelGGL(k_build_index, dim3(frames), dim3(kIndexThreads), lds, stream, coords,
                       offs, frame_begin, H, W, K, n_rows, tok_base, N, M, err);
    return hipGetLastError();
}

}  // namespace svc
