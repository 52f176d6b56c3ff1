// Neighbour index table on the GPU ("SV-TAD: Native Sparse Convolutions for
// Efficient Temporal Action Detection", Key Design 1: the lookup map M and
// the neighbour table N, both O(N_kept)).
//
// One workgroup per frame.  The frame's map lives in LDS (H*W int32, at most
// 64 KiB): fill with -1, scatter M[p_k] = k with an atomic exchange (a
// previous value other than -1 means two tokens on one cell), then each
// thread produces consecutive elements of the frame's contiguous N block, so
// the rows (K*K int32 each) are written fully coalesced.  The coordinates
// are requested before the map is filled and kept in LDS for both steps.  The neighbourhood
// is K x K (K odd), tap j = K (dy + K/2) + (dx + K/2) for offsets dy, dx in
// [-K/2, K/2]: the 3 x 3 case is the one the page builds.
#include "internal.h"

namespace svc {

constexpr int kIndexThreads = 256;
// Frames of at most this many cells also keep their tokens' cells in LDS
// (map and cells together within 64 KiB).
constexpr int kCacheCells = 8192;

// K: side of the neighbourhood (compile time, so that the row / tap split of
// a table element is a multiplication).  CACHE: the frame's token cells are
// read once, before the map is filled, and kept in LDS as (y << 16) | x;
// without it (frames of more than kCacheCells cells) they are read from
// memory again for the table.
template <int K, bool CACHE>
__global__ __launch_bounds__(kIndexThreads) void k_build_index(
    const int32_t* __restrict__ coords, const int32_t* __restrict__ offs, int frame_begin,
    int H, int W, int64_t n_rows, int64_t tok_base, int32_t* __restrict__ N,
    int32_t* __restrict__ M, int32_t* __restrict__ err) {
    constexpr int taps = K * K, rad = K / 2;
    extern __shared__ int32_t smem[];
    const int cells = H * W;
    int32_t* smap = smem;
    int32_t* syx = smem + cells;               // CACHE: token r of the frame -> (y << 16) | x, -1 if out of range
    const int t = frame_begin + static_cast<int>(blockIdx.x);
    const int64_t beg = offs[t], end = offs[t + 1];
    int flag = 0;
    // The frame's rows must lie inside the caller's N buffer.
    const bool ok = beg >= tok_base && end >= beg && end - tok_base <= n_rows &&
                    end - beg <= cells;
    if (!ok) flag |= SV_FLAG_BAD_OFFSETS;
    // ... and the frames together must cover all n_rows of it: the first
    // frame starts at row 0 and the last ends at row n_rows (rows outside
    // every frame would be left unwritten).
    if (blockIdx.x == 0 && beg != tok_base) flag |= SV_FLAG_BAD_OFFSETS;
    if (blockIdx.x == gridDim.x - 1 && end != tok_base + n_rows) flag |= SV_FLAG_BAD_OFFSETS;
    const int cnt = ok ? static_cast<int>(end - beg) : 0;
    const int32_t* __restrict__ cf = coords + beg;

    if constexpr (CACHE) {
        for (int r = threadIdx.x; r < cnt; r += kIndexThreads) {
            const int p = cf[r];
            int yx = -1;
            if (static_cast<unsigned>(p) < static_cast<unsigned>(cells)) {
                const int y = p / W;
                yx = (y << 16) | (p - y * W);
            } else {
                flag |= SV_FLAG_COORD_RANGE;
            }
            syx[r] = yx;
        }
    }
    for (int c = threadIdx.x; c < cells; c += kIndexThreads) smap[c] = -1;
    __syncthreads();

    // Step 1: M[p_k] = k (indices relative to tok_base).
    for (int r = threadIdx.x; r < cnt; r += kIndexThreads) {
        int p;
        if constexpr (CACHE) {
            const int yx = syx[r];
            if (yx < 0) continue;
            p = (yx >> 16) * W + (yx & 0xffff);
        } else {
            p = cf[r];
            if (static_cast<unsigned>(p) >= static_cast<unsigned>(cells)) {
                flag |= SV_FLAG_COORD_RANGE;
                continue;
            }
        }
        const int old = atomicExch(&smap[p], static_cast<int>(beg + r - tok_base));
        if (old != -1) flag |= SV_FLAG_DUPLICATE;
    }
    __syncthreads();

    // Step 2: N[k][j] = M[y + dy_j][x + dx_j], bounds checked per axis; each
    // thread writes consecutive elements of the frame's contiguous N block.
    {
        const int total = cnt * taps;   // <= 16384 * 49
        int32_t* __restrict__ Nf = N + (beg - tok_base) * taps;
        for (int e = threadIdx.x; e < total; e += kIndexThreads) {
            const int r = e / taps;
            const int j = e - r * taps;
            int y = -1, x = 0;
            if constexpr (CACHE) {
                const int yx = syx[r];
                if (yx >= 0) {
                    y = yx >> 16;
                    x = yx & 0xffff;
                }
            } else {
                const int p = cf[r];
                if (static_cast<unsigned>(p) < static_cast<unsigned>(cells)) {
                    y = p / W;
                    x = p - y * W;
                }
            }
            int v = -1;
            if (y >= 0) {
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

template <int K>
static void launch_index_k(dim3 grid, bool cache, size_t cells, hipStream_t stream, const int32_t* coords,
                           const int32_t* offs, int frame_begin, int H, int W, int64_t n_rows, int64_t tok_base,
                           int32_t* N, int32_t* M, int32_t* err) {
    if (cache)
        hipLaunchKernelGGL((k_build_index<K, true>), grid, dim3(kIndexThreads), 2 * cells * sizeof(int32_t), stream,
                           coords, offs, frame_begin, H, W, n_rows, tok_base, N, M, err);
    else
        hipLaunchKernelGGL((k_build_index<K, false>), grid, dim3(kIndexThreads), cells * sizeof(int32_t), stream,
                           coords, offs, frame_begin, H, W, n_rows, tok_base, N, M, err);
}

hipError_t launch_build_index(const int32_t* coords, const int32_t* offs, int frame_begin,
                              int frames, int H, int W, int K, int64_t n_rows, int64_t tok_base,
                              int32_t* N, int32_t* M, int32_t* err, hipStream_t stream) {
    if (frames <= 0) return hipSuccess;
    const size_t cells = static_cast<size_t>(H) * W;
    const bool cache = cells <= static_cast<size_t>(kCacheCells);
    const dim3 grid(frames);
    switch (K) {
    case 1: launch_index_k<1>(grid, cache, cells, stream, coords, offs, frame_begin, H, W, n_rows, tok_base, N, M, err); break;
    case 3: launch_index_k<3>(grid, cache, cells, stream, coords, offs, frame_begin, H, W, n_rows, tok_base, N, M, err); break;
    case 5: launch_index_k<5>(grid, cache, cells, stream, coords, offs, frame_begin, H, W, n_rows, tok_base, N, M, err); break;
    case 7: launch_index_k<7>(grid, cache, cells, stream, coords, offs, frame_begin, H, W, n_rows, tok_base, N, M, err); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace svc
