/*
 * svconv -- native SparseConv2D on pruned token sequences, HIP for gfx950.
 *
 * C ABI.  Plain pointers and sizes only; every pointer argument named "device"
 * is device memory owned by the caller; the library never allocates, never
 * frees, never synchronises the stream (unless the SV_SYNC_CHECK debugging
 * aid below is switched on, sv_sparseconv2d_chunked is given no host copy
 * of the frame offsets, or in sv_sparseconv2d_chunked_host, which orders its
 * copy engines from the host) and keeps no state other than a cached device
 * property.  All work is enqueued asynchronously on the caller's
 * hipStream_t (NULL = the default stream).  No C++ exception crosses this
 * boundary.  Status codes report argument errors synchronously, before any
 * work is enqueued; data errors found on the device (coordinates) are OR-ed
 * into a caller-provided device flag.
 *
 * The method ("SV-TAD: Native Sparse Convolutions for Efficient Temporal
 * Action Detection", paper notes page):
 *   - Key Design 1 (Static Neighbor Index Table): a per-frame lookup map M of
 *     H x W cells set to -1, then M[y_k, x_k] = k for every kept token; the
 *     neighbour table N [n x 9] reads M at the nine 3x3 offsets, -1 where the
 *     neighbour was pruned or falls outside the grid.
 *   - Key Design 2 (Native Sparse 2D Convolution Kernels): y_k =
 *     sum_j W_j x[N[k, j]], an entry of -1 acting as zero padding, computed
 *     directly on the packed token sequence; chunked execution keeps memory
 *     independent of video length.
 *
 * Conventions used throughout:
 *   tap j = 3*(dy+1) + (dx+1), dy, dx in {-1,0,1}; centre tap j = 4.
 *   Cross-correlation: tap j of token k reads the token at (y+dy, x+dx).
 *   Flat coordinate p = y * W + x.  Tokens are packed frame-major; frame t
 *   owns tokens frame_offsets[t] .. frame_offsets[t+1]-1.
 *   Row-major contiguous layouts:
 *     X [n][C_in], Y [n][C_out], N [n][9] int32 (global packed indices),
 *     Wt [9][C_in][C_out]  (Wt[j][i][o] = torch weight[o][i][j/3][j%3]),
 *     bias [C_out] (same dtype as X), dW [9][C_in][C_out] fp32, db [C_out] fp32.
 *   bf16 = IEEE binary32 truncated to its upper 16 bits; outputs rounded to
 *   nearest even.  Accumulation is always fp32.
 */
#ifndef SVCONV_H
#define SVCONV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sv_status {
    SV_OK = 0,
    SV_ERR_INVALID_ARG = 1,     /* null pointer, negative size, bad combination   */
    SV_ERR_UNSUPPORTED = 2,     /* dtype / shape not supported by the kernel asked */
    SV_ERR_WORKSPACE = 3,       /* workspace missing or smaller than required      */
    SV_ERR_HIP = 4,             /* a HIP launch or query failed                   */
    SV_ERR_COORD_RANGE = 5,     /* (device flag bit 1) coordinate outside H x W    */
    SV_ERR_DUPLICATE_COORD = 6  /* (device flag bit 2) two tokens on one cell      */
} sv_status;

typedef enum sv_dtype { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

/* Kernel choice for the convolution passes.  AUTO picks the bf16 MFMA kernel
 * when dtype is bf16, C_in % 32 == 0 and C_out % 16 == 0 (dX: the same with
 * C_in and C_out swapped) and the gathered input (n x contracted channels
 * bf16) spans at most 2 GiB, and the VALU kernel otherwise.  The weight and
 * bias gradients use the MFMA kernel under the same size bound with both
 * channel counts multiples of 128. */
typedef enum sv_kernel { SV_KERNEL_AUTO = 0, SV_KERNEL_VALU = 1, SV_KERNEL_MFMA = 2 } sv_kernel;

/* Bits of the device error flag written by sv_build_index. */
#define SV_FLAG_COORD_RANGE   1  /* a coordinate p < 0 or p >= H*W                        */
#define SV_FLAG_DUPLICATE     2  /* two tokens of one frame on one cell                   */
#define SV_FLAG_BAD_OFFSETS   4  /* frame_offsets not non-decreasing from 0 to exactly n   */

/* Passes of sv_sparseconv2d_chunked. */
#define SV_PASS_FWD 1u
#define SV_PASS_DX  2u
#define SV_PASS_DW  4u

/* Operations for sv_workspace_bytes. */
typedef enum sv_op { SV_OP_FWD = 0, SV_OP_DX = 1, SV_OP_DW = 2 } sv_op;

/* ------------------------------------------------------------------------ */
/* Key Design 1, both steps, on the GPU: per frame the map M lives in LDS
 * (one workgroup per frame), is filled with -1, receives M[p_k] = k by atomic
 * exchange (a second token on one cell raises SV_FLAG_DUPLICATE), and the
 * nine lookups write N with bounds checked on y and x separately.
 *
 *   coords        device int32 [n]   flat coordinate of each kept token
 *   frame_offsets device int32 [T+1] exclusive prefix sums of tokens per frame
 *   T, H, W       frames and grid; H*W <= 16384 (LDS map), T >= 0
 *   n             number of tokens = length of coords = rows of N_out
 *   N_out         device int32 [n][9], written
 *   M_out         nullable; device int32 [T][H][W], written with token
 *                 indices (-1 for pruned cells)
 *   err_flag      nullable; device int32, SV_FLAG_* bits OR-ed in (never
 *                 cleared by the library).  Tokens with a bad coordinate get
 *                 an all -1 row; with duplicates N is unspecified.
 * Returns SV_ERR_INVALID_ARG for null required pointers or bad sizes,
 * SV_ERR_UNSUPPORTED for H*W > 16384.
 *
 * Debugging aid: with SV_SYNC_CHECK=1 in the environment (read at every
 * call), this call and the chunk drivers wait for their stream after
 * enqueuing and return the status the device flag implies (SV_ERR_COORD_RANGE,
 * SV_ERR_DUPLICATE_COORD, or SV_ERR_INVALID_ARG for SV_FLAG_BAD_OFFSETS).
 * The flag is never cleared by the library, so earlier bits count too.
 * Without the variable nothing here synchronises. */
sv_status sv_build_index(const int32_t *coords, const int32_t *frame_offsets,
                         int32_t T, int32_t H, int32_t W, int64_t n,
                         int32_t *N_out, int32_t *M_out, int32_t *err_flag,
                         hipStream_t stream);

/* Key Design 2, forward: Y[k][o] = sum_j sum_i X[N[k,j]][i] Wt[j][i][o]
 * + bias[o]; entries of N that are -1 (or outside [0, n)) contribute zero.
 *   X [n][C_in], N [n][9], Wt [9][C_in][C_out], bias [C_out] nullable,
 *   Y [n][C_out] written; all device, all in `dtype` except N.
 *   workspace: device, 16-byte aligned, at least
 *   sv_workspace_bytes(SV_OP_FWD, ...) bytes (0 unless the bf16 matrix-core
 *   kernels can run; it receives the weights repacked for them: as
 *   [tap][C_out][C_in], or in MFMA fragment order when C_in is a multiple of
 *   64 and C_out of 128); contents are scratch.
 * SV_ERR_UNSUPPORTED if `kernel` is MFMA and the shape/dtype does not fit it;
 * SV_ERR_WORKSPACE if the MFMA kernel runs and the workspace is short. */
sv_status sv_sparseconv2d_fwd(const void *X, const int32_t *N, const void *Wt,
                              const void *bias, void *Y, int64_t n,
                              int32_t C_in, int32_t C_out, sv_dtype dtype,
                              sv_kernel kernel, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* Key Design 2's dedicated backward kernels, input gradient.  The page
 * prints no backward formula; this is the adjoint of the forward sum,
 * written as gathers thanks to the mirrored offsets (token m is tap j of k
 * exactly when k is tap 8-j of m):
 *   dX[k][i] = sum_j sum_o dY[N[k,8-j]][o] Wt[j][i][o].
 *   dY [n][C_out], N [n][9], Wt [9][C_in][C_out], dX [n][C_in] written.
 *   workspace: device, nullable.  When the bf16 matrix-core path runs on a
 *   shape whose weights it takes in fragment order (C_out a multiple of 64,
 *   C_in of 128) and Wt is 16-byte aligned, a workspace of at least
 *   sv_workspace_bytes(SV_OP_DX, ...) bytes (16-byte aligned) receives the
 *   repacked weights and the faster kernel runs; without one the kernel that
 *   reads Wt directly runs.  Both give the same bits.
 * SV_ERR_UNSUPPORTED if `kernel` is MFMA and the shape/dtype does not fit it;
 * SV_ERR_WORKSPACE if a workspace is given but is short. */
sv_status sv_sparseconv2d_bwd_dx(const void *dY, const int32_t *N, const void *Wt,
                                 void *dX, int64_t n, int32_t C_in, int32_t C_out,
                                 sv_dtype dtype, sv_kernel kernel, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* Weight (and bias) gradient, a split-K reduction over tokens ("SV-TAD:
 * Native Sparse Convolutions for Efficient Temporal Action Detection",
 * Key Design 2: the method has dedicated backward kernels; the page prints
 * no backward formula, and this one is the adjoint of the forward sum):
 *   dW[j][i][o] (+)= sum_k X[N[k,j]][i] dY[k][o],   db[o] (+)= sum_k dY[k][o].
 * Token slices write fp32 partials to the workspace, then a fixed-order
 * reduction adds them (deterministic: the same inputs give the same bits).
 *   X [n][C_in], N [n][9], dY [n][C_out] in `dtype`;
 *   dW [9][C_in][C_out] fp32 device, written (accumulate == 0) or added to;
 *   db [C_out] fp32 device, nullable, same accumulate rule;
 *   workspace: device, at least sv_workspace_bytes(SV_OP_DW, ...) bytes,
 *   16-byte aligned; its contents are scratch. */
sv_status sv_sparseconv2d_bwd_dw(const void *X, const int32_t *N, const void *dY,
                                 float *dW, float *db, int64_t n, int32_t C_in,
                                 int32_t C_out, sv_dtype dtype, int32_t accumulate,
                                 void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Workspace bytes an operation needs for these sizes (FWD: the repacked
 * weights of the bf16 matrix-core kernels, else 0; DX: the fragment-order
 * weights where the input gradient takes them, else 0; DW: token-slice
 * partials).  Depends only on its arguments, never on the device. */
size_t sv_workspace_bytes(sv_op op, int64_t n, int32_t C_in, int32_t C_out, sv_dtype dtype);

/* K x K neighbourhoods.  The five calls above for any odd K in {1, 3, 5, 7}
 * (they are these with K = 3).  With taps = K*K and r = K/2:
 *   tap j = K*(dy + r) + (dx + r), dy, dx in [-r, r]; centre tap taps/2;
 *   tap taps-1-j is the mirror (-dy, -dx) of tap j, so the input gradient
 *   reads Wt[taps-1-j] where the 3 x 3 case reads Wt[8-j];
 *   N [n][taps], Wt and dW [taps][C_in][C_out]
 *   (Wt[j][i][o] = torch weight[o][i][j/K][j%K]).
 * The page ("SV-TAD: Native Sparse Convolutions for Efficient Temporal
 * Action Detection", Key Design 2) builds the 3 x 3 convolution of its
 * adapter; K = 1 is the pointwise projection around it (N[k][0] = k) and
 * 5 and 7 widen the receptive field with the same index table and
 * kernels.  Both kernel families serve every K listed; the MFMA conditions
 * of sv_kernel are unchanged, and the fragment-order weights (workspaces
 * of FWD and DX) apply at K = 3, 5 and 7 (at K = 1 from 512 contracted
 * channels).  n * taps must stay below 2^31.
 * Returns SV_ERR_INVALID_ARG for an even or non-positive K and
 * SV_ERR_UNSUPPORTED for an odd K above 7 (sv_workspace_bytes_k: 0), then
 * behaves exactly as the 3 x 3 call of the same name. */
sv_status sv_build_index_k(const int32_t *coords, const int32_t *frame_offsets,
                           int32_t T, int32_t H, int32_t W, int32_t K, int64_t n,
                           int32_t *N_out, int32_t *M_out, int32_t *err_flag,
                           hipStream_t stream);
sv_status sv_sparseconv2d_fwd_k(const void *X, const int32_t *N, const void *Wt,
                                const void *bias, void *Y, int64_t n, int32_t K,
                                int32_t C_in, int32_t C_out, sv_dtype dtype,
                                sv_kernel kernel, void *workspace, size_t workspace_bytes,
                                hipStream_t stream);
sv_status sv_sparseconv2d_bwd_dx_k(const void *dY, const int32_t *N, const void *Wt,
                                   void *dX, int64_t n, int32_t K, int32_t C_in, int32_t C_out,
                                   sv_dtype dtype, sv_kernel kernel, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream);
sv_status sv_sparseconv2d_bwd_dw_k(const void *X, const int32_t *N, const void *dY,
                                   float *dW, float *db, int64_t n, int32_t K, int32_t C_in,
                                   int32_t C_out, sv_dtype dtype, int32_t accumulate,
                                   void *workspace, size_t workspace_bytes,
                                   hipStream_t stream);
size_t sv_workspace_bytes_k(sv_op op, int64_t n, int32_t K, int32_t C_in, int32_t C_out,
                            sv_dtype dtype);

/* Split forms, for callers that schedule the pieces of a training step
 * themselves (same definitions as above; Key Design 2's forward and
 * dedicated backward kernels):
 *   sv_repack_fwd_k writes the forward's repacked weights
 *     V[taps-1-j][o][i] = Wt[j][i][o] (bf16 only; V device, 16-byte aligned,
 *     at least sv_workspace_bytes_k(SV_OP_FWD, ...) bytes for a shape the
 *     MFMA kernel takes), and sv_sparseconv2d_fwd_packed_k runs the forward
 *     on the MFMA kernel from that V (SV_ERR_UNSUPPORTED where the kernel does
 *     not fit).  Weights repacked once serve any number of forward calls and
 *     can be prepared on another stream ahead of them.
 *   sv_repack_dx_k writes the input gradient's weights in MFMA fragment
 *     order (bf16, K of 3, 5 or 7, or K = 1 with C_out of at least 512;
 *     C_out a multiple of 64 and C_in of 128; else
 *     SV_ERR_UNSUPPORTED; Wt and P 16-byte aligned, P at least
 *     sv_workspace_bytes_k(SV_OP_DX, ...) bytes), and
 *     sv_sparseconv2d_bwd_dx_packed_k runs the input gradient from that P;
 *     the pair equals sv_sparseconv2d_bwd_dx_k bit for bit.
 *   sv_sparseconv2d_bwd_dw_partials_k then sv_sparseconv2d_bwd_dw_reduce_k,
 *     with the same arguments and workspace and in this order (the second
 *     may run on another stream once the first has finished), equal one
 *     sv_sparseconv2d_bwd_dw_k call bit for bit: the first writes the token
 *     slices' partials into the workspace (or dW and db themselves with one
 *     slice), the second adds them in fixed order.  db must be given to both
 *     or to neither.  The workspace stays in use until the second completes. */
sv_status sv_repack_fwd_k(const void *Wt, int32_t K, int32_t C_in, int32_t C_out, sv_dtype dtype,
                          void *V, size_t V_bytes, hipStream_t stream);
sv_status sv_sparseconv2d_fwd_packed_k(const void *X, const int32_t *N, const void *V,
                                       const void *bias, void *Y, int64_t n, int32_t K,
                                       int32_t C_in, int32_t C_out, sv_dtype dtype,
                                       hipStream_t stream);
/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the weight
 * gradient of sv_sparseconv2d_bwd_dw_k with its token-slice partials kept in
 * a device array of the library instead of a caller workspace.  Same
 * arguments as sv_sparseconv2d_bwd_dw_k minus the workspace, same plan,
 * kernels and summation order, so the same bits.
 *   The array holds SV_NOALLOC_SCRATCH_BYTES bytes on every GPU the library
 *   runs on, from module load until the process ends; it is found (with
 *   hipGetSymbolAddress) on the first call on each device, which must be the
 *   current device of the calling thread and the device of `stream`.
 *   Shapes whose partials exceed it (sv_workspace_bytes_k(SV_OP_DW, ...) >
 *   SV_NOALLOC_SCRATCH_BYTES) return SV_ERR_WORKSPACE.
 *   All calls on one GPU share that GPU's array and it keeps the last call's
 *   contents (nothing in it needs to start at zero): calls that may overlap
 *   on one GPU -- on different streams, or from different threads without
 *   ordering -- race, and must be ordered by the caller.
 * Allocates nothing and never synchronises; SV_ERR_HIP if the device or the
 * array cannot be found. */
#define SV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
sv_status sv_sparseconv2d_bwd_dw_noalloc_k(const void *X, const int32_t *N, const void *dY,
                                           float *dW, float *db, int64_t n, int32_t K,
                                           int32_t C_in, int32_t C_out, sv_dtype dtype,
                                           int32_t accumulate, hipStream_t stream);

sv_status sv_repack_dx_k(const void *Wt, int32_t K, int32_t C_in, int32_t C_out, sv_dtype dtype,
                         void *P, size_t P_bytes, hipStream_t stream);
/* The repacks of several layers of one shape in a single launch, for a
 * step that repacks every layer's weights up front (Key Design 2's forward
 * and backward kernels consume them): for i < count (1..16), V[i] receives
 * what sv_repack_fwd_k(Wt[i], ...) writes and P[i] what sv_repack_dx_k(Wt[i],
 * ...) writes.  Wt, V, P: host arrays of device pointers; V or P may be
 * NULL (that layout is not written), but not their entries; every V[i]
 * holds V_bytes and every P[i] P_bytes (16-byte aligned; each at least
 * sv_workspace_bytes_k(SV_OP_FWD / SV_OP_DX, ...)).  bf16 only; P needs a
 * shape sv_repack_dx_k takes (else SV_ERR_UNSUPPORTED). */
sv_status sv_repack_layers_k(int32_t count, const void *const *Wt, void *const *V, size_t V_bytes,
                             void *const *P, size_t P_bytes, int32_t K, int32_t C_in, int32_t C_out,
                             sv_dtype dtype, hipStream_t stream);
sv_status sv_sparseconv2d_bwd_dx_packed_k(const void *dY, const int32_t *N, const void *P, void *dX,
                                          int64_t n, int32_t K, int32_t C_in, int32_t C_out,
                                          sv_dtype dtype, hipStream_t stream);
sv_status sv_sparseconv2d_bwd_dw_partials_k(const void *X, const int32_t *N, const void *dY,
                                            float *dW, float *db, int64_t n, int32_t K,
                                            int32_t C_in, int32_t C_out, sv_dtype dtype,
                                            int32_t accumulate, void *workspace,
                                            size_t workspace_bytes, hipStream_t stream);
sv_status sv_sparseconv2d_bwd_dw_reduce_k(float *dW, float *db, int64_t n, int32_t K, int32_t C_in,
                                          int32_t C_out, sv_dtype dtype, int32_t accumulate,
                                          const void *workspace, size_t workspace_bytes,
                                          hipStream_t stream);

/* Chunked execution over whole frames (Key Design 2's chunking): the frames
 * are processed chunk_frames at a time; for each chunk the index table is
 * built with chunk-local indices into the workspace, then the requested
 * passes run on the chunk's token range.  Spatial neighbourhoods never cross
 * frames, so chunks need no halo and the results equal the unchunked ones
 * (N shifted by the chunk base; Y and dX identical; dW/db summed over chunks
 * in chunk order).  Workspace is sized by the largest chunk, not by T. */
typedef struct sv_chunked_desc {
    int32_t T, H, W;
    int32_t C_in, C_out;
    sv_dtype dtype;
    sv_kernel kernel;
    int32_t chunk_frames;               /* >= 1                                  */
    const int32_t *coords;              /* device [n]                            */
    const int32_t *frame_offsets;       /* device [T+1]                          */
    const int32_t *frame_offsets_host;  /* host [T+1], the same values, or NULL:
                                           the call then copies frame_offsets to
                                           the host and waits for that copy on
                                           `stream` (it needs the chunk
                                           boundaries to size its launches), and
                                           the workspace is sized for chunks of
                                           chunk_frames full frames (H*W tokens
                                           each) */
    const void *X;                      /* device [n][C_in]   (FWD, DW)          */
    const void *Wt;                     /* device [9][C_in][C_out] (FWD, DX)     */
    const void *bias;                   /* device [C_out], nullable              */
    void *Y;                            /* device [n][C_out]  (FWD)              */
    const void *dY;                     /* device [n][C_out]  (DX, DW)           */
    void *dX;                           /* device [n][C_in]   (DX)               */
    float *dW;                          /* device [9][C_in][C_out] fp32 (DW), overwritten */
    float *db;                          /* device [C_out] fp32, nullable (DW), overwritten */
    int32_t *err_flag;                  /* device int32, nullable                */
    int32_t ksize;                      /* K of a K x K neighbourhood (the _k calls);
                                           0 selects 3.  N, Wt, dW then hold K*K taps */
    hipStream_t dw_stream;              /* nullable.  With the DW pass and FWD or DX,
                                           each chunk's dW + db runs on this stream,
                                           concurrently with the next chunks' index
                                           builds and convolutions on the call's
                                           stream.  It first waits for the work
                                           enqueued on the call's stream before the
                                           call, and the call's stream waits for it
                                           at the end, so on the call's stream the
                                           results are complete in stream order and
                                           bit-identical to the one-stream run.  The
                                           workspace then holds a second N table
                                           (sv_chunked_workspace_bytes counts it).
                                           The call's own stream here means the
                                           one-stream run. */
} sv_chunked_desc;

sv_status sv_sparseconv2d_chunked(const sv_chunked_desc *desc, uint32_t passes,
                                  void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* Workspace bytes sv_sparseconv2d_chunked needs for this descriptor (reads
 * only the host fields: T, H, W, C_in, C_out, dtype, chunk_frames,
 * frame_offsets_host, ksize; with frame_offsets_host NULL, the bound for
 * chunks of full frames, which covers any offsets).  Returns 0 and nothing
 * else on bad descriptors.  sv_sparseconv2d_chunked returns SV_ERR_UNSUPPORTED for an
 * odd ksize above 7 and SV_ERR_INVALID_ARG for other bad ones. */
size_t sv_chunked_workspace_bytes(const sv_chunked_desc *desc, uint32_t passes);

/* Host-streamed chunked execution: the chunk driver above with the
 * per-token tensors left in host memory ("SV-TAD: Native Sparse
 * Convolutions for Efficient Temporal Action Detection", Key Design 2:
 * chunking decouples memory from the length of the video; here the device
 * holds only the weights, the gradients and a workspace sized by one chunk,
 * so total device memory does not grow with T).
 *
 * Each chunk's coordinates, frame offsets, X and dY are copied by the copy
 * engines (hipMemcpyAsync) into one of four device staging sets on `h2d`,
 * computed on `compute` (index build, then the requested passes, exactly as
 * sv_sparseconv2d_chunked), and its Y and dX copied back on `d2h`.  Uploads
 * run two chunks ahead of the compute, and a chunk's results go back while
 * the next chunks compute.  The copy streams never wait on another stream's
 * event (a copy queued behind such a wait can hold the host thread in the
 * runtime until it fires); the call orders them from the host instead: it
 * waits (on the host) for a chunk's compute before queuing its download,
 * and for a staging set's download before queuing the next upload into it.
 * So, unlike the other calls, this one blocks the host: it returns once the
 * last chunk's compute has finished and its download is queued.  Results
 * are identical to sv_sparseconv2d_chunked (same kernels, same chunk order;
 * dW/db accumulate on the device in chunk order).
 *
 * All host arrays must be page-locked (hipHostMalloc, or a pinned torch
 * tensor; anything else is SV_ERR_INVALID_ARG) and must stay valid, and
 * Y / dX unread, until `compute` completes: the call makes `compute` wait
 * for the last copies, so synchronising `compute` suffices.  The three
 * streams must be distinct.  The call first waits (on the host) for the
 * work already enqueued on `compute`, so back-to-back calls on one workspace
 * are ordered.  It creates (and releases) thirteen HIP events; it allocates
 * no memory.  On a HIP error part of the work may already be enqueued. */
typedef struct sv_chunked_host_desc {
    int32_t T, H, W;
    int32_t C_in, C_out;
    sv_dtype dtype;
    sv_kernel kernel;
    int32_t chunk_frames;               /* >= 1                                  */
    const int32_t *coords_host;         /* pinned host [n]                       */
    const int32_t *frame_offsets_host;  /* pinned host [T+1]                     */
    const void *X_host;                 /* pinned host [n][C_in]  (FWD, DW)      */
    const void *Wt;                     /* device [9][C_in][C_out] (FWD, DX)     */
    const void *bias;                   /* device [C_out], nullable              */
    void *Y_host;                       /* pinned host [n][C_out] (FWD)          */
    const void *dY_host;                /* pinned host [n][C_out] (DX, DW)       */
    void *dX_host;                      /* pinned host [n][C_in]  (DX)           */
    float *dW;                          /* device [9][C_in][C_out] fp32 (DW), overwritten */
    float *db;                          /* device [C_out] fp32, nullable (DW), overwritten */
    int32_t *err_flag;                  /* device int32, nullable                */
    int32_t ksize;                      /* as in sv_chunked_desc: 0 selects 3    */
} sv_chunked_host_desc;

sv_status sv_sparseconv2d_chunked_host(const sv_chunked_host_desc *desc, uint32_t passes,
                                       void *workspace, size_t workspace_bytes,
                                       hipStream_t compute, hipStream_t h2d, hipStream_t d2h);

/* Workspace bytes sv_sparseconv2d_chunked_host needs: the device driver's
 * workspace plus four staging sets of the largest chunk's coordinates,
 * offsets and per-token tensors.  Independent of T.  Returns 0 on bad
 * descriptors. */
size_t sv_chunked_host_workspace_bytes(const sv_chunked_host_desc *desc, uint32_t passes);

/* Bottleneck adapter ("SV-TAD: Native Sparse Convolutions for Efficient
 * Temporal Action Detection", Overall Architecture and Key Design 3: lightweight
 * bottleneck adapters run on the pruned tokens; the visual features inside
 * them are down-projected).  The page prints no further internals; read as
 * the plain residual bottleneck
 *   H1 = X Wd + bd                    down-projection C -> r (a 1 x 1 SparseConv2D)
 *   H2 = SparseConv2D_KxK(H1) + bc    r -> r over the neighbour table N
 *   Y  = X + H2 Wu + bu               up-projection r -> C; the residual is
 *                                     added in the projection's kernel,
 *                                     before its one rounding
 * with no activation (the page names none).  Layouts, row-major, all in
 * `dtype` except N: X, Y [n][C]; N [n][K*K] (sv_build_index_k);
 * Wd [C][r] (a [1][C][r] weight), Wc [K*K][r][r], Wu [r][C]; biases bd [r],
 * bc [r], bu [C], each nullable; H1, H2 [n][r] written, kept for the
 * backward (H1 is also what the cross-attention below attends over).
 * The three layers run the kernels of the calls above (MFMA when `kernel`
 * and the shapes allow, per layer; SV_ERR_UNSUPPORTED if MFMA is forced and
 * a layer does not fit), in order on `stream`.  Workspace:
 * sv_adapter_workspace_bytes(0, ...) bytes, 256-byte aligned (an identity
 * table for the projections and the repacked weights).  K as in the _k
 * calls. */
sv_status sv_adapter_fwd(const void *X, const int32_t *N, int64_t n, int32_t K, int32_t C, int32_t r,
                         const void *Wd, const void *bd, const void *Wc, const void *bc,
                         const void *Wu, const void *bu, void *H1, void *H2, void *Y,
                         sv_dtype dtype, sv_kernel kernel, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Adapter backward for an upstream gradient dY [n][C], given the forward's
 * H1 and H2:
 *   dWu = H2^T dY,  dbu = sum_k dY[k];      dH2 = dY Wu^T
 *   dWc, dbc = the K x K weight gradient of (H1, dH2);  dH1 = its input gradient
 *   dWd = X^T dH1,  dbd = sum_k dH1[k];     dX  = dY + dH1 Wd^T
 * (the last sum in one kernel, before its one rounding).  dW* and db* are
 * fp32, overwritten; db* nullable.  dH2 and dH1 are held in the workspace in
 * `dtype` (sv_adapter_workspace_bytes(1, ...) bytes, 256-byte aligned), with
 * the weight-gradient partials and the input gradients' weights repacked in
 * fragment order where the bf16 matrix-core kernel takes them.
 * Deterministic.
 * dw_stream (nullable; the call's own stream means the same): the three
 * weight gradients run on it, each after the tensor it reads is ready on
 * `stream`, beside the input gradients on `stream`; `stream` waits for it at
 * the end, so on `stream` every output is complete in stream order and
 * bit-identical to the one-stream run. */
sv_status sv_adapter_bwd(const void *X, const int32_t *N, int64_t n, int32_t K, int32_t C, int32_t r,
                         const void *Wd, const void *Wc, const void *Wu,
                         const void *H1, const void *H2, const void *dY,
                         void *dX, float *dWd, float *dbd, float *dWc, float *dbc,
                         float *dWu, float *dbu, sv_dtype dtype, sv_kernel kernel,
                         void *workspace, size_t workspace_bytes, hipStream_t stream,
                         hipStream_t dw_stream);
/* Workspace bytes of sv_adapter_fwd (backward == 0) or sv_adapter_bwd;
 * 0 for invalid sizes.  Depends only on the arguments. */
size_t sv_adapter_workspace_bytes(int32_t backward, int64_t n, int32_t K, int32_t C, int32_t r,
                                  sv_dtype dtype);

/* Asymmetric cross-attention (Key Design 3): auxiliary tokens Q [m][d]
 * (such as the CLS token) query the down-projected sparse visual tokens
 * X [n][d], which serve as keys and as values; only the auxiliary tokens are
 * updated.  Read as single-head scaled dot-product attention with no further
 * projections:
 *   S[q][j] = scale * <Q[q], X[j]>,   O[q] = sum_j softmax_j(S[q])[j] X[j],
 *   lse[q]  = log sum_j exp(S[q][j])  (-inf when n == 0, where O = 0).
 * scale == 0 selects 1/sqrt(d).  d is 64, 128 or 256 (else
 * SV_ERR_UNSUPPORTED); m <= 65535.  Q, X, O, dO, dX: device, `dtype`,
 * row-major, 16-byte aligned; lse and dQ: device fp32.  To attend within one
 * frame chunk only, pass that chunk's rows of X.
 *
 * Forward: O [m][d] and lse [m] written.  Split over key blocks; the
 * partials go to the workspace (sv_xattn_workspace_bytes(0, m, n, d) bytes,
 * 16-byte aligned) and are merged in block order: deterministic.
 *
 * Backward for an upstream gradient dO [m][d], given the forward's O and
 * lse: dQ [m][d] (fp32) and dX [n][d] written, with
 *   D[q]     = sum_j P[q][j] <dO[q], X[j]>   (summed over the keys)
 *   dS[q][j] = P[q][j] (<dO[q], X[j]> - D[q]),
 *   dQ[q]    = scale sum_j dS[q][j] X[j],
 *   dX[j]    = scale sum_q dS[q][j] Q[q] + sum_q P[q][j] dO[q]
 * (X enters as keys and as values).  O only shifts the keys inside these
 * sums (dS sums to zero over the keys, so the result is the same for any
 * shift in exact arithmetic); shifting by the softmax-weighted mean keeps
 * fp32 accurate when the tokens share a large component.  Two passes over
 * X.  Workspace sv_xattn_workspace_bytes(1, m, n, d) bytes.  With m == 0,
 * dX is zeroed. */
sv_status sv_xattn_fwd(const void *Q, const void *X, int64_t m, int64_t n, int32_t d,
                       float scale, sv_dtype dtype, void *O, float *lse,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);
sv_status sv_xattn_bwd(const void *Q, const void *X, const void *O, const void *dO,
                       const float *lse, int64_t m, int64_t n, int32_t d, float scale,
                       sv_dtype dtype, float *dQ, void *dX,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);
/* Workspace bytes of sv_xattn_fwd (backward == 0) or sv_xattn_bwd
 * (backward != 0); 0 for unsupported sizes.  Depends only on the arguments. */
size_t sv_xattn_workspace_bytes(int32_t backward, int64_t m, int64_t n, int32_t d);

/* Stage transition between pruning stages (the map is rebuilt at each
 * selection point and reused by the adapter layers in between, Key Design 1):
 * the next stage's packed input keeps a subset of the current rows.
 *   sv_stage_gather:  dst[r] = src[rows[r]]            for r < n_rows
 *   sv_stage_scatter: dst[m] = 0 for every m < n_dst, then dst[rows[r]] = src[r]
 * (the backward of the gather).  Rows are C elements of `dtype`; rows[] is
 * device int32 [n_rows]; for the scatter rows[] must be distinct; an index
 * outside [0, n_src) / [0, n_dst) skips that row. */
sv_status sv_stage_gather(const void *src, int64_t n_src, const int32_t *rows,
                          int64_t n_rows, void *dst, int32_t C, sv_dtype dtype,
                          hipStream_t stream);
sv_status sv_stage_scatter(const void *src, const int32_t *rows, int64_t n_rows,
                           void *dst, int64_t n_dst, int32_t C, sv_dtype dtype,
                           hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char *sv_status_string(sv_status status);

/* Library version, e.g. "svconv 0.1.0 gfx950". */
const char *sv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SVCONV_H */
