// Stage transitions between pruning stages: the next stage keeps a subset of
// the current packed rows ("SV-TAD: Native Sparse Convolutions for Efficient
// Temporal Action Detection", Overall Architecture and Key Design 1: tokens
// are re-selected at fixed layers and the index table is rebuilt there).
// Pure row copies, bound by HBM bandwidth: one thread per 16-byte (or 4- or
// 2-byte) word of a row.
#include "internal.h"

namespace svc {

template <typename V>
__global__ __launch_bounds__(256) void k_gather_rows(const V* __restrict__ src, int64_t n_src,
                                                     const int32_t* __restrict__ rows, int64_t n_rows,
                                                     V* __restrict__ dst, int words) {
    const int64_t total = n_rows * words;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total; e += stride) {
        const int64_t r = e / words;
        const int w = static_cast<int>(e - r * words);
        const int64_t m = rows[r];
        if (m >= 0 && m < n_src) dst[e] = src[m * words + w];
    }
}

template <typename V>
__global__ __launch_bounds__(256) void k_fill_zero(V* __restrict__ dst, int64_t count) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < count; e += stride)
        dst[e] = V{};
}

template <typename V>
__global__ __launch_bounds__(256) void k_scatter_rows(const V* __restrict__ src,
                                                      const int32_t* __restrict__ rows, int64_t n_rows,
                                                      V* __restrict__ dst, int64_t n_dst, int words) {
    const int64_t total = n_rows * words;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total; e += stride) {
        const int64_t r = e / words;
        const int w = static_cast<int>(e - r * words);
        const int64_t m = rows[r];
        if (m >= 0 && m < n_dst) dst[m * words + w] = src[e];
    }
}

static unsigned blocks_for(int64_t work) {
    int64_t b = (work + 255) / 256;
    return static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>(b, 8192)));
}

template <typename V>
static hipError_t gather_as(const void* src, int64_t n_src, const int32_t* rows, int64_t n_rows, void* dst,
                            int words, hipStream_t stream) {
    hipLaunchKernelGGL(k_gather_rows<V>, dim3(blocks_for(n_rows * words)), dim3(256), 0, stream,
                       static_cast<const V*>(src), n_src, rows, n_rows, static_cast<V*>(dst), words);
    return hipGetLastError();
}

template <typename V>
static hipError_t scatter_as(const void* src, const int32_t* rows, int64_t n_rows, void* dst, int64_t n_dst,
                             int words, hipStream_t stream) {
    hipLaunchKernelGGL(k_fill_zero<V>, dim3(blocks_for(n_dst * words)), dim3(256), 0, stream,
                       static_cast<V*>(dst), n_dst * words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n_rows == 0) return e;
    hipLaunchKernelGGL(k_scatter_rows<V>, dim3(blocks_for(n_rows * words)), dim3(256), 0, stream,
                       static_cast<const V*>(src), rows, n_rows, static_cast<V*>(dst), n_dst, words);
    return hipGetLastError();
}

static bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

hipError_t launch_stage_gather(const void* src, int64_t n_src, const int32_t* rows, int64_t n_rows, void* dst,
                               int C, int elem_bytes, hipStream_t stream) {
    if (n_rows <= 0) return hipSuccess;
    const int64_t rb = static_cast<int64_t>(C) * elem_bytes;
    if (rb % 16 == 0 && aligned(src, 16) && aligned(dst, 16))
        return gather_as<uint4>(src, n_src, rows, n_rows, dst, static_cast<int>(rb / 16), stream);
    if (rb % 4 == 0 && aligned(src, 4) && aligned(dst, 4))
        return gather_as<uint32_t>(src, n_src, rows, n_rows, dst, static_cast<int>(rb / 4), stream);
    return gather_as<uint16_t>(src, n_src, rows, n_rows, dst, static_cast<int>(rb / 2), stream);
}

hipError_t launch_stage_scatter(const void* src, const int32_t* rows, int64_t n_rows, void* dst, int64_t n_dst,
                                int C, int elem_bytes, hipStream_t stream) {
    if (n_dst <= 0) return hipSuccess;
    const int64_t rb = static_cast<int64_t>(C) * elem_bytes;
    if (rb % 16 == 0 && aligned(src, 16) && aligned(dst, 16))
        return scatter_as<uint4>(src, rows, n_rows, dst, n_dst, static_cast<int>(rb / 16), stream);
    if (rb % 4 == 0 && aligned(src, 4) && aligned(dst, 4))
        return scatter_as<uint32_t>(src, rows, n_rows, dst, n_dst, static_cast<int>(rb / 4), stream);
    return scatter_as<uint16_t>(src, rows, n_rows, dst, n_dst, static_cast<int>(rb / 2), stream);
}

// The identity neighbour table of a 1 x 1 neighbourhood: dst[k] = k.
__global__ __launch_bounds__(256) void k_iota(int32_t* __restrict__ dst, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t k = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; k < n; k += stride)
        dst[k] = static_cast<int32_t>(k);
}

hipError_t launch_iota(int32_t* dst, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int blocks = static_cast<int>(std::min<int64_t>((n + 255) / 256, 1024));
    hipLaunchKernelGGL(k_iota, dim3(blocks), dim3(256), 0, stream, dst, n);
    return hipGetLastError();
}

}  // namespace svc
