// Internal declarations shared by the HIP translation units of libsvconv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "svconv.h"

namespace svc {

// ---------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest, ties to even; NaN stays NaN (quiet bit set).  This is
// gfx950's conversion instruction (v_cvt_pk_bf16_f32), which produces exactly
// those bits -- (u + 0x7fff + ((u >> 16) & 1)) >> 16 for a non-NaN pattern u,
// (u >> 16) | 0x40 for a NaN -- for every one of the 2^32 fp32 inputs
// (compared on the GPU).  One instruction, where the bit arithmetic took ten
// and a per-value branch for the NaN test took more: an epilogue rounds 128
// values per lane.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float* p) { return *p; }
    static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<uint16_t> {
    static __device__ __forceinline__ float load(const uint16_t* p) { return bf16_to_f32(*p); }
    static __device__ __forceinline__ void store(uint16_t* p, float v) { *p = f32_to_bf16(v); }
};

// A row of N is valid when 0 <= m < n; anything else reads as zero padding.
__device__ __forceinline__ int clamp_index(int m, int n) {
    return (static_cast<unsigned>(m) < static_cast<unsigned>(n)) ? m : -1;
}

// Raw buffer loads: a 128-bit resource (base, byte range) in scalar
// registers, 32-bit per-lane byte offsets, and the hardware range check: a
// load at an offset at or past the range returns zeros and makes no memory
// request.  kOob is such an offset for every range used here (all ranges are
// at most 2^31 bytes; callers check that on the host).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOob = 0x80000000u;
constexpr uint32_t kMaxRange = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    // dword 3 = 0x00020000: untyped 32-bit data format, the CDNA default
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 load16(rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ int load4(rsrc_t r, uint32_t off) {
    return static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Workgroups of a 1-D grid go to the 8 XCDs of the chip round-robin by
// linear id, and each XCD has its own L2.  This maps the linear id to a
// logical tile id so that every XCD receives one contiguous range of logical
// tiles, in order: tiles that share inputs (neighbouring token ranges, the
// output-channel tiles of one token range) then run on the same XCD at about
// the same time and meet their shared rows in its L2.  Bijective on [0, count).
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_remap(int linear, int count) {
    const int xcd = linear % kXcds, local = linear / kXcds;
    const int base = count / kXcds, extra = count % kXcds;
    return xcd * base + min(xcd, extra) + local;
}

// ---------------------------------------------------------------- launchers
// Every launcher enqueues on `stream` and returns hipGetLastError().

// K: side of the K x K neighbourhood (odd); N rows hold K * K entries.
hipError_t launch_build_index(const int32_t* coords, const int32_t* offs, int frame_begin,
                              int frames, int H, int W, int K, int64_t n, int64_t tok_base,
                              int32_t* N, int32_t* M, int32_t* err, hipStream_t stream);

// In the conv launchers `taps` = K * K: the columns of N and the leading
// dimension of the weights; tap taps-1-j is the mirror of tap j.
//
// Both paths add an optional residual R (nullable, shaped like the output)
// before the single rounding of the output.
//
// VALU path (fp32 or bf16, any channel count).  `dx` selects the input
// gradient: A = dY [n][Co], output [n][Ci], weights read transposed with the
// tap mirrored; otherwise A = X [n][Ci], output [n][Co].
hipError_t launch_conv_valu(bool bf16, bool dx, const void* A, const int32_t* N,
                            const void* Wt, const void* bias, const void* R, void* out, int64_t n,
                            int Ci, int Co, int taps, hipStream_t stream);

// MFMA path (bf16, taps in {1, 9, 25, 49}).  One gather-GEMM serves both
// passes:
//   out[k][c] = sum_j sum_i A[N[k,j]][i] * B[taps-1-j][c][i] (+ bias[c]),
// A [n][K], B [taps][NO][K] (K % 32 == 0, NO % 16 == 0).  The input gradient
// calls it with A = dY and B = Wt; the forward with A = X and B = V, the
// weights repacked by launch_repack_fwd (V[taps-1-j][o][i] = Wt[j][i][o])
// into conv_mfma_fwd_workspace(Ci, Co, taps) bytes.
hipError_t launch_conv_mfma_packed(const uint16_t* A, const int32_t* N, const uint16_t* B,
                                   const uint16_t* bias, const uint16_t* R, uint16_t* out, int64_t n, int K,
                                   int NO, int taps, hipStream_t stream);
// Two problems on the same N in one launch: (A1, B1, bias1) -> out1 and
// (A2, B2) -> out2, each as launch_conv_mfma_packed (no residual).  The
// chunk driver runs a chunk's forward and input gradient together this way.
hipError_t launch_conv_mfma_pair(const uint16_t* A1, const uint16_t* B1, const uint16_t* bias1, uint16_t* out1,
                                 int K1, int NO1, const uint16_t* A2, const uint16_t* B2, uint16_t* out2, int K2,
                                 int NO2, const int32_t* N, int64_t n, int taps, hipStream_t stream);
// allow_frag = false keeps the per-tap layout even where the fragment-order
// kernel could run (a call with a residual, which only k_conv_mfma takes).
hipError_t launch_repack_fwd(const uint16_t* Wt, uint16_t* V, int Ci, int Co, int taps, hipStream_t stream,
                             bool allow_frag = true);
// Weight operand in fragment order (conv_bfrag.hip): the MFMA kernel that
// streams B from memory into registers.  conv_bfrag_ok: the shapes it is
// built for (3 x 3, 5 x 5, 7 x 7 or 1 x 1, contracted channels a multiple of
// 64, produced channels a multiple of 128); conv_bfrag_pair_ok: those its
// paired launch takes (3 x 3 and 1 x 1).  The repack writes taps * Ci * Co bf16 in fragment
// order for the forward (dx = false: K = Ci, NO = Co) or the input gradient
// (dx = true: K = Co, NO = Ci, taps mirrored).
bool conv_bfrag_ok(int K, int NO, int taps);
bool conv_bfrag_pair_ok(int K1, int NO1, int K2, int NO2, int taps);
hipError_t launch_repack_frag(const uint16_t* Wt, uint16_t* Bf, int Ci, int Co, int taps, bool dx,
                              hipStream_t stream);
// Up to kRepackMax layers' weights (Wt[i], all of one shape) into both
// fragment orders in one launch: V[i] for the forward, P[i] for the input
// gradient (V, P or their entries nullable); the shapes must suit
// conv_bfrag_ok for each layout written.
constexpr int kRepackMax = 16;
hipError_t launch_repack_batch(int count, const uint16_t* const* W, uint16_t* const* V, uint16_t* const* P, int Ci,
                               int Co, int taps, hipStream_t stream);
hipError_t launch_conv_bfrag(const uint16_t* A, const int32_t* N, const uint16_t* Bf, const uint16_t* bias,
                             uint16_t* out, int64_t n, int K, int NO, int taps, hipStream_t stream);
// Two problems on the same N in one launch, each as launch_conv_bfrag (the
// second without bias): the shapes must suit conv_bfrag_pair_ok.  slots:
// the workgroups the tile shape may count on (kBfragSlots, one per compute
// unit, or fewer to leave room for a kernel on another stream).
constexpr int kBfragSlots = 256;
hipError_t launch_conv_bfrag_pair(const uint16_t* A1, const uint16_t* B1, const uint16_t* bias1, uint16_t* out1,
                                  int K1, int NO1, const uint16_t* A2, const uint16_t* B2, uint16_t* out2, int K2,
                                  int NO2, const int32_t* N, int64_t n, int taps, int slots, hipStream_t stream);
size_t conv_mfma_fwd_workspace(int Ci, int Co, int taps);
// bf16, a tap count the kernel is built for, contracted channels a multiple
// of 32, output channels of 16, and the n rows of A and of the output within
// the 2 GiB range of a buffer load.
bool conv_mfma_supported(bool dx, int Ci, int Co, int64_t n, int taps);

// dW: split-K plan, partial kernels, reduction.
struct DwPlan {
    int taps;              // K * K
    bool mfma;
    int slices;            // token slices (split-K factor)
    int64_t slice_tokens;  // tokens per slice (multiple of the kernel's token step)
    size_t partial_floats; // floats of dW partials in the workspace (0 when slices == 1)
    size_t db_floats;      // floats of db partials
};
DwPlan plan_dw(int64_t n, int Ci, int Co, bool bf16, int taps);
size_t dw_workspace_bytes(const DwPlan& p);
hipError_t launch_dw(const DwPlan& plan, bool bf16, const void* X, const int32_t* N,
                     const void* dY, float* dW, float* db, int64_t n, int Ci, int Co,
                     int accumulate, void* ws, hipStream_t stream);
// The two phases of launch_dw, for callers that put them on different
// streams: the partial kernels, then the fixed-order reduction of the
// workspace they wrote (same plan, dW, db and workspace).
hipError_t launch_dw_partials(const DwPlan& plan, bool bf16, const void* X, const int32_t* N,
                              const void* dY, float* dW, float* db, int64_t n, int Ci, int Co,
                              int accumulate, void* ws, hipStream_t stream);
hipError_t launch_dw_reduce(const DwPlan& plan, float* dW, float* db, int Ci, int Co, int accumulate,
                            const void* ws, hipStream_t stream);

// Asymmetric cross-attention: key blocks of kpb keys, partials in the
// workspace (fwd_bytes / bwd_bytes), head width d in {64, 128, 256}.
struct XattnPlan {
    int64_t kpb;       // keys per block (a multiple of 16)
    int64_t blocks;    // key blocks
    size_t fwd_bytes;  // workspace of the forward
    size_t bwd_bytes;  // workspace of the backward
};
XattnPlan plan_xattn(int64_t m, int64_t n, int d);
bool xattn_supported(int d);
hipError_t launch_xattn_fwd(const XattnPlan& p, bool bf16, const void* Q, const void* X, int m, int64_t n, int d,
                            float scale, void* O, float* lse, void* ws, hipStream_t stream);
hipError_t launch_xattn_bwd(const XattnPlan& p, bool bf16, const void* Q, const void* X, const void* O,
                            const void* dO, const float* lse, int m, int64_t n, int d, float scale, float* dQ,
                            void* dX, void* ws, hipStream_t stream);

// Dense 1 x 1 layer with a residual, Y = A B + bias + R (bf16; K in {64,
// 128, 256} contracted channels, Co a multiple of 256): B repacked into
// fragment order (dense_res_ws_bytes) from W = B (trans = false, [K][Co]) or
// W = B^T (trans = true, [Co][K]); bias and R nullable.
bool dense_res_supported(bool bf16, int K, int Co, int64_t n);
size_t dense_res_ws_bytes(int K, int Co);
hipError_t launch_repack_dense(const uint16_t* W, uint16_t* Bf, int K, int Co, bool trans, hipStream_t stream);
hipError_t launch_dense_res(const uint16_t* A, const uint16_t* Bf, const uint16_t* bias, const uint16_t* R,
                            uint16_t* Y, int64_t n, int K, int Co, hipStream_t stream);

hipError_t launch_stage_gather(const void* src, int64_t n_src, const int32_t* rows, int64_t n_rows,
                               void* dst, int C, int elem_bytes, hipStream_t stream);
hipError_t launch_stage_scatter(const void* src, const int32_t* rows, int64_t n_rows, void* dst,
                                int64_t n_dst, int C, int elem_bytes, hipStream_t stream);
// dst[k] = k for k < n: the neighbour table of a 1 x 1 neighbourhood.
hipError_t launch_iota(int32_t* dst, int64_t n, hipStream_t stream);

}  // namespace svc
