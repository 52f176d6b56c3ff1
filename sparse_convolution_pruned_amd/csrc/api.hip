// C ABI of libsvconv: argument validation, kernel dispatch, chunk driver.
// Nothing here allocates or synchronises; every launch goes to the caller's
// stream.  Declarations and contracts: include/svconv.h.
#include <limits>

#include <vector>

#include "internal.h"

#include <cmath>
#include <cstdlib>

using namespace svc;

namespace {

constexpr int kMaxCells = 16384;
constexpr int kMaxK = 7;

// Rows of N: n * taps int32 entries must stay addressable with 32-bit
// element indices.
int64_t max_rows(int taps) { return std::numeric_limits<int32_t>::max() / taps; }

// taps = K * K for a supported odd K; SV_ERR_INVALID_ARG for an even or
// non-positive K, SV_ERR_UNSUPPORTED for odd K > kMaxK.
sv_status taps_of(int32_t K, int* taps) {
    if (K < 1 || K % 2 == 0) return SV_ERR_INVALID_ARG;
    if (K > kMaxK) return SV_ERR_UNSUPPORTED;
    *taps = K * K;
    return SV_OK;
}

bool valid_dtype(sv_dtype d) { return d == SV_F32 || d == SV_BF16; }

// Opt-in check for debugging (SV_SYNC_CHECK=1 in the environment, read at
// every call): after enqueuing an index build the call waits for its stream
// and turns the bits of the device error flag into a status.  The flag
// accumulates, so a bit set by an earlier call is reported again.
sv_status sync_check(const int32_t* err_flag, hipStream_t stream) {
    const char* e = getenv("SV_SYNC_CHECK");
    if (!err_flag || !e || e[0] != '1') return SV_OK;
    int32_t f = 0;
    if (hipMemcpyAsync(&f, err_flag, sizeof(f), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return SV_ERR_HIP;
    if (f & SV_FLAG_BAD_OFFSETS) return SV_ERR_INVALID_ARG;
    if (f & SV_FLAG_COORD_RANGE) return SV_ERR_COORD_RANGE;
    if (f & SV_FLAG_DUPLICATE) return SV_ERR_DUPLICATE_COORD;
    return SV_OK;
}
bool valid_kernel(sv_kernel k) { return k == SV_KERNEL_AUTO || k == SV_KERNEL_VALU || k == SV_KERNEL_MFMA; }
sv_status hip_status(hipError_t e) { return e == hipSuccess ? SV_OK : SV_ERR_HIP; }
size_t align_up(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// Which conv kernel runs a pass; SV_ERR_UNSUPPORTED when MFMA is forced and
// does not fit.
sv_status choose(sv_kernel req, sv_dtype dt, bool dx, int Ci, int Co, int64_t n, int taps, bool* use_mfma) {
    const bool fits = dt == SV_BF16 && conv_mfma_supported(dx, Ci, Co, n, taps);
    if (req == SV_KERNEL_MFMA && !fits) return SV_ERR_UNSUPPORTED;
    *use_mfma = (req == SV_KERNEL_MFMA) || (req == SV_KERNEL_AUTO && fits);
    return SV_OK;
}

sv_status conv_args_ok(int64_t n, int taps, int32_t Ci, int32_t Co, sv_dtype dt, sv_kernel k) {
    if (n < 0 || n > max_rows(taps) || Ci <= 0 || Co <= 0) return SV_ERR_INVALID_ARG;
    if (!valid_dtype(dt) || !valid_kernel(k)) return SV_ERR_INVALID_ARG;
    return SV_OK;
}

// Forward with the repacked weights already in `V` (MFMA path) or straight
// from Wt (VALU path); R: nullable residual added to Y.
sv_status run_fwd_prepared(bool mfma, const void* X, const int32_t* N, const void* Wt, const void* V,
                           const void* bias, void* Y, int64_t n, int32_t Ci, int32_t Co, int taps,
                           sv_dtype dt, hipStream_t s, const void* R = nullptr) {
    if (n == 0) return SV_OK;
    if (mfma && !R && conv_bfrag_ok(Ci, Co, taps)) {
        // V holds the weights in fragment order (launch_repack_fwd); a call
        // with a residual has them in the per-tap layout for k_conv_mfma
        return hip_status(launch_conv_bfrag(static_cast<const uint16_t*>(X), N, static_cast<const uint16_t*>(V),
                                            static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(Y), n, Ci, Co,
                                            taps, s));
    }
    if (mfma)
        return hip_status(launch_conv_mfma_packed(static_cast<const uint16_t*>(X), N,
                                                  static_cast<const uint16_t*>(V),
                                                  static_cast<const uint16_t*>(bias),
                                                  static_cast<const uint16_t*>(R),
                                                  static_cast<uint16_t*>(Y), n, Ci, Co, taps, s));
    return hip_status(launch_conv_valu(dt == SV_BF16, false, X, N, Wt, bias, R, Y, n, Ci, Co, taps, s));
}

// Input gradient; R: nullable residual added to dX.  P: nullable, the
// weights in fragment order for the input gradient (launch_repack_frag with
// dx = true), used when the fragment kernel takes the shape; without it the
// MFMA path reads Wt directly.
sv_status run_dx(const void* dY, const int32_t* N, const void* Wt, void* dX, int64_t n, int32_t Ci,
                 int32_t Co, int taps, sv_dtype dt, sv_kernel kernel, hipStream_t s, const void* R = nullptr,
                 const void* P = nullptr) {
    bool mfma = false;
    sv_status st = choose(kernel, dt, true, Ci, Co, n, taps, &mfma);
    if (st != SV_OK) return st;
    if (n == 0) return SV_OK;
    if (mfma && P && !R && conv_bfrag_ok(Co, Ci, taps))
        return hip_status(launch_conv_bfrag(static_cast<const uint16_t*>(dY), N, static_cast<const uint16_t*>(P),
                                            nullptr, static_cast<uint16_t*>(dX), n, Co, Ci, taps, s));
    if (mfma)
        return hip_status(launch_conv_mfma_packed(static_cast<const uint16_t*>(dY), N,
                                                  static_cast<const uint16_t*>(Wt), nullptr,
                                                  static_cast<const uint16_t*>(R),
                                                  static_cast<uint16_t*>(dX), n, Co, Ci, taps, s));
    return hip_status(launch_conv_valu(dt == SV_BF16, true, dY, N, Wt, nullptr, R, dX, n, Ci, Co, taps, s));
}

// Forward and input gradient of one chunk, both on the MFMA kernels, in one
// paired launch where one kernel takes both shapes: k_conv_bfrag with V and
// P in fragment order, else k_conv_mfma (the forward from the repacked
// weights V, the input gradient from Wt).  The two problems' tiles fill the
// chip together.
sv_status run_fwd_dx_pair(const void* X, const void* dY, const int32_t* N, const void* Wt, const void* V,
                          const void* P, const void* bias, void* Y, void* dX, int64_t n, int32_t Ci, int32_t Co,
                          int taps, int slots, hipStream_t s) {
    if (n == 0) return SV_OK;
    if (P && conv_bfrag_pair_ok(Ci, Co, Co, Ci, taps))
        // both passes on the fragment kernel (V and P in fragment order)
        return hip_status(launch_conv_bfrag_pair(static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(V),
                                                 static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(Y), Ci,
                                                 Co, static_cast<const uint16_t*>(dY),
                                                 static_cast<const uint16_t*>(P), static_cast<uint16_t*>(dX), Co,
                                                 Ci, N, n, taps, slots, s));
    if (conv_bfrag_ok(Ci, Co, taps) || conv_bfrag_ok(Co, Ci, taps)) {
        // fragment-order weights for one of the passes: each runs on its own launch
        sv_status st = run_fwd_prepared(true, X, N, Wt, V, bias, Y, n, Ci, Co, taps, SV_BF16, s);
        if (st != SV_OK) return st;
        return run_dx(dY, N, Wt, dX, n, Ci, Co, taps, SV_BF16, SV_KERNEL_MFMA, s, nullptr, P);
    }
    return hip_status(launch_conv_mfma_pair(static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(V),
                                            static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(Y), Ci, Co,
                                            static_cast<const uint16_t*>(dY), static_cast<const uint16_t*>(Wt),
                                            static_cast<uint16_t*>(dX), Co, Ci, N, n, taps, s));
}

// Bytes of repacked weights the forward needs when the MFMA kernel may run.
size_t fwd_ws_bytes(int32_t Ci, int32_t Co, sv_dtype dt, int64_t n, int taps) {
    return (dt == SV_BF16 && conv_mfma_supported(false, Ci, Co, n, taps)) ? conv_mfma_fwd_workspace(Ci, Co, taps)
                                                                           : 0;
}

// Bytes of fragment-order weights the input gradient takes when the
// fragment kernel can run it (same size as the forward's repack), else 0.
size_t dx_ws_bytes(int32_t Ci, int32_t Co, sv_dtype dt, int64_t n, int taps) {
    return (dt == SV_BF16 && conv_mfma_supported(true, Ci, Co, n, taps) && conv_bfrag_ok(Co, Ci, taps))
               ? conv_mfma_fwd_workspace(Ci, Co, taps)
               : 0;
}

}  // namespace

extern "C" {

sv_status sv_build_index_k(const int32_t* coords, const int32_t* frame_offsets, int32_t T, int32_t H,
                           int32_t W, int32_t K, int64_t n, int32_t* N_out, int32_t* M_out, int32_t* err_flag,
                           hipStream_t stream) {
    int taps = 0;
    sv_status st = taps_of(K, &taps);
    if (st != SV_OK) return st;
    if (T < 0 || H <= 0 || W <= 0 || n < 0 || n > max_rows(taps)) return SV_ERR_INVALID_ARG;
    if (!frame_offsets || (n > 0 && (!coords || !N_out))) return SV_ERR_INVALID_ARG;
    if (static_cast<int64_t>(H) * W > kMaxCells) return SV_ERR_UNSUPPORTED;
    if (T == 0) return SV_OK;
    if ((st = hip_status(launch_build_index(coords, frame_offsets, 0, T, H, W, K, n, 0, N_out, M_out, err_flag,
                                            stream))) != SV_OK)
        return st;
    return sync_check(err_flag, stream);
}

sv_status sv_build_index(const int32_t* coords, const int32_t* frame_offsets, int32_t T, int32_t H,
                         int32_t W, int64_t n, int32_t* N_out, int32_t* M_out, int32_t* err_flag,
                         hipStream_t stream) {
    return sv_build_index_k(coords, frame_offsets, T, H, W, 3, n, N_out, M_out, err_flag, stream);
}

sv_status sv_sparseconv2d_fwd_k(const void* X, const int32_t* N, const void* Wt, const void* bias, void* Y,
                                int64_t n, int32_t K, int32_t C_in, int32_t C_out, sv_dtype dtype,
                                sv_kernel kernel, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int taps = 0;
    sv_status st = taps_of(K, &taps);
    if (st != SV_OK) return st;
    if ((st = conv_args_ok(n, taps, C_in, C_out, dtype, kernel)) != SV_OK) return st;
    if (!Wt || (n > 0 && (!X || !N || !Y))) return SV_ERR_INVALID_ARG;
    bool mfma = false;
    if ((st = choose(kernel, dtype, false, C_in, C_out, n, taps, &mfma)) != SV_OK) return st;
    if (mfma) {
        const size_t need = conv_mfma_fwd_workspace(C_in, C_out, taps);
        if (!workspace || workspace_bytes < need) return SV_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(workspace) % 16) return SV_ERR_INVALID_ARG;
        if (n == 0) return SV_OK;
        st = hip_status(launch_repack_fwd(static_cast<const uint16_t*>(Wt), static_cast<uint16_t*>(workspace),
                                          C_in, C_out, taps, stream));
        if (st != SV_OK) return st;
    }
    return run_fwd_prepared(mfma, X, N, Wt, workspace, bias, Y, n, C_in, C_out, taps, dtype, stream);
}

sv_status sv_sparseconv2d_fwd(const void* X, const int32_t* N, const void* Wt, const void* bias,
                              void* Y, int64_t n, int32_t C_in, int32_t C_out, sv_dtype dtype,
                              sv_kernel kernel, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    return sv_sparseconv2d_fwd_k(X, N, Wt, bias, Y, n, 3, C_in, C_out, dtype, kernel, workspace,
                                 workspace_bytes, stream);
}

sv_status sv_sparseconv2d_bwd_dx_k(const void* dY, const int32_t* N, const void* Wt, void* dX, int64_t n,
                                   int32_t K, int32_t C_in, int32_t C_out, sv_dtype dtype, sv_kernel kernel,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int taps = 0;
    sv_status st = taps_of(K, &taps);
    if (st != SV_OK) return st;
    if ((st = conv_args_ok(n, taps, C_in, C_out, dtype, kernel)) != SV_OK) return st;
    if (!Wt || (n > 0 && (!dY || !N || !dX))) return SV_ERR_INVALID_ARG;
    bool mfma = false;
    if ((st = choose(kernel, dtype, true, C_in, C_out, n, taps, &mfma)) != SV_OK) return st;
    const size_t need = dx_ws_bytes(C_in, C_out, dtype, n, taps);
    // The repack reads Wt in 16-byte pieces; a Wt that is not 16-byte
    // aligned takes the kernel that reads it directly.
    if (mfma && need > 0 && workspace && reinterpret_cast<uintptr_t>(Wt) % 16 == 0) {
        if (workspace_bytes < need) return SV_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(workspace) % 16) return SV_ERR_INVALID_ARG;
        if (n == 0) return SV_OK;
        st = hip_status(launch_repack_frag(static_cast<const uint16_t*>(Wt), static_cast<uint16_t*>(workspace),
                                           C_in, C_out, taps, true, stream));
        if (st != SV_OK) return st;
        return run_dx(dY, N, Wt, dX, n, C_in, C_out, taps, dtype, kernel, stream, nullptr, workspace);
    }
    return run_dx(dY, N, Wt, dX, n, C_in, C_out, taps, dtype, kernel, stream);
}

sv_status sv_sparseconv2d_bwd_dx(const void* dY, const int32_t* N, const void* Wt, void* dX,
                                 int64_t n, int32_t C_in, int32_t C_out, sv_dtype dtype,
                                 sv_kernel kernel, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return sv_sparseconv2d_bwd_dx_k(dY, N, Wt, dX, n, 3, C_in, C_out, dtype, kernel, workspace, workspace_bytes,
                                    stream);
}

size_t sv_workspace_bytes_k(sv_op op, int64_t n, int32_t K, int32_t C_in, int32_t C_out, sv_dtype dtype) {
    int taps = 0;
    if (taps_of(K, &taps) != SV_OK) return 0;
    if (n < 0 || C_in <= 0 || C_out <= 0 || !valid_dtype(dtype)) return 0;
    if (op == SV_OP_FWD) return fwd_ws_bytes(C_in, C_out, dtype, n, taps);
    if (op == SV_OP_DX) return dx_ws_bytes(C_in, C_out, dtype, n, taps);
    if (op != SV_OP_DW) return 0;
    return dw_workspace_bytes(plan_dw(n, C_in, C_out, dtype == SV_BF16, taps));
}

size_t sv_workspace_bytes(sv_op op, int64_t n, int32_t C_in, int32_t C_out, sv_dtype dtype) {
    return sv_workspace_bytes_k(op, n, 3, C_in, C_out, dtype);
}

sv_status sv_sparseconv2d_bwd_dw_k(const void* X, const int32_t* N, const void* dY, float* dW, float* db,
                                   int64_t n, int32_t K, int32_t C_in, int32_t C_out, sv_dtype dtype,
                                   int32_t accumulate, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
    int taps = 0;
    sv_status st = taps_of(K, &taps);
    if (st != SV_OK) return st;
    if ((st = conv_args_ok(n, taps, C_in, C_out, dtype, SV_KERNEL_AUTO)) != SV_OK) return st;
    if (!dW || (n > 0 && (!X || !N || !dY))) return SV_ERR_INVALID_ARG;
    const DwPlan plan = plan_dw(n, C_in, C_out, dtype == SV_BF16, taps);
    const size_t need = dw_workspace_bytes(plan);
    if (need > 0 && (!workspace || workspace_bytes < need)) return SV_ERR_WORKSPACE;
    if (workspace && reinterpret_cast<uintptr_t>(workspace) % 16) return SV_ERR_INVALID_ARG;
    return hip_status(launch_dw(plan, dtype == SV_BF16, X, N, dY, dW, db, n, C_in, C_out,
                                accumulate ? 1 : 0, workspace, stream));
}

sv_status sv_sparseconv2d_bwd_dw(const void* X, const int32_t* N, const void* dY, float* dW, float* db,
                                 int64_t n, int32_t C_in, int32_t C_out, sv_dtype dtype,
                                 int32_t accumulate, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
    return sv_sparseconv2d_bwd_dw_k(X, N, dY, dW, db, n, 3, C_in, C_out, dtype, accumulate, workspace,
                                    workspace_bytes, stream);
}

// ------------------------------------------- split forms for scheduling
sv_status sv_repack_fwd_k(const void* Wt, int32_t K, int32_t C_in, int32_t C_out, sv_dtype dtype, void* V,
                          size_t V_bytes, hipStream_t stream) {
    int taps = 0;
    sv_status st = taps_of(K, &taps);
    if (st != SV_OK) return st;
    if (C_in <= 0 || C_out <= 0 || !valid_dtype(dtype) || !Wt || !V) return SV_ERR_INVALID_ARG;
    if (dtype != SV_BF16) return SV_ERR_UNSUPPORTED;
    if (V_bytes < conv_mfma_fwd_workspace(C_in, C_out, taps)) return SV_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(V) % 16) return SV_ERR_INVALID_ARG;
    return hip_status(launch_repack_fwd(static_cast<const uint16_t*>(Wt), static_cast<uint16_t*>(V), C_in, C_out,
                                        taps, stream));
}

sv_status sv_sparseconv2d_fwd_packed_k(const void* X, const int32_t* N, const void* V, const void* bias, void* Y,
                                       int64_t n, int32_t K, int32_t C_in, int32_t C_out, sv_dtype dtype,
                                       hipStream_t stream) {
    int taps = 0;
    sv_status st = taps_of(K, &taps);
    if (st != SV_OK) return st;
    if ((st = conv_args_ok(n, taps, C_in, C_out, dtype, SV_KERNEL_MFMA)) != SV_OK) return st;
    if (!V || (n > 0 && (!X || !N || !Y))) return SV_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(V) % 16) return SV_ERR_INVALID_ARG;
    bool mfma = false;
    if ((st = choose(SV_KERNEL_MFMA, dtype, false, C_in, C_out, n, taps, &mfma)) != SV_OK) return st;
    return run_fwd_prepared(true, X, N, nullptr, V, bias, Y, n, C_in, C_out, taps, dtype, stream);
}

sv_status sv_repack_dx_k(const void* Wt, int32_t K, int32_t C_in, int32_t C_out, sv_dtype dtype, void* P,
                         size_t P_bytes, hipStream_t stream) {
    int taps = 0;
    sv_status st = taps_of(K, &taps);
    if (st != SV_OK) return st;
    if (C_in <= 0 || C_out <= 0 || !valid_dtype(dtype) || !Wt || !P) return SV_ERR_INVALID_ARG;
    if (dtype != SV_BF16 || !conv_bfrag_ok(C_out, C_in, taps)) return SV_ERR_UNSUPPORTED;
    if (P_bytes < conv_mfma_fwd_workspace(C_in, C_out, taps)) return SV_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(P) % 16 || reinterpret_cast<uintptr_t>(Wt) % 16) return SV_ERR_INVALID_ARG;
    return hip_status(launch_repack_frag(static_cast<const uint16_t*>(Wt), static_cast<uint16_t*>(P), C_in, C_out,
                                         taps, true, stream));
}

sv_status sv_repack_layers_k(int32_t count, const void* const* Wt, void* const* V, size_t V_bytes, void* const* P,
                             size_t P_bytes, int32_t K, int32_t C_in, int32_t C_out, sv_dtype dtype,
                             hipStream_t stream) {
    int taps = 0;
    sv_status st = taps_of(K, &taps);
    if (st != SV_OK) return st;
    if (count < 1 || count > kRepackMax || !Wt || C_in <= 0 || C_out <= 0 || !valid_dtype(dtype))
        return SV_ERR_INVALID_ARG;
    if (dtype != SV_BF16) return SV_ERR_UNSUPPORTED;
    const size_t need = conv_mfma_fwd_workspace(C_in, C_out, taps);
    for (int i = 0; i < count; ++i) {
        if (!Wt[i] || (V && !V[i]) || (P && !P[i])) return SV_ERR_INVALID_ARG;
        if ((V && reinterpret_cast<uintptr_t>(V[i]) % 16) || (P && reinterpret_cast<uintptr_t>(P[i]) % 16))
            return SV_ERR_INVALID_ARG;
    }
    if (V && (!conv_mfma_supported(false, C_in, C_out, 1, taps))) return SV_ERR_UNSUPPORTED;
    if (P && !conv_bfrag_ok(C_out, C_in, taps)) return SV_ERR_UNSUPPORTED;
    if ((V && V_bytes < need) || (P && P_bytes < need)) return SV_ERR_WORKSPACE;
    const bool vfrag = V && conv_bfrag_ok(C_in, C_out, taps);
    auto W16 = reinterpret_cast<const uint16_t* const*>(Wt);
    if (vfrag || P) {
        st = hip_status(launch_repack_batch(count, W16, vfrag ? reinterpret_cast<uint16_t* const*>(V) : nullptr,
                                            reinterpret_cast<uint16_t* const*>(P), C_in, C_out, taps, stream));
        if (st != SV_OK) return st;
    }
    if (V && !vfrag)
        for (int i = 0; i < count; ++i)
            if ((st = hip_status(launch_repack_fwd(W16[i], static_cast<uint16_t*>(V[i]), C_in, C_out, taps, stream))) !=
                SV_OK)
                return st;
    return SV_OK;
}

sv_status sv_sparseconv2d_bwd_dx_packed_k(const void* dY, const int32_t* N, const void* P, void* dX, int64_t n,
                                          int32_t K, int32_t C_in, int32_t C_out, sv_dtype dtype,
                                          hipStream_t stream) {
    int taps = 0;
    sv_status st = taps_of(K, &taps);
    if (st != SV_OK) return st;
    if ((st = conv_args_ok(n, taps, C_in, C_out, dtype, SV_KERNEL_MFMA)) != SV_OK) return st;
    if (!P || (n > 0 && (!dY || !N || !dX))) return SV_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(P) % 16) return SV_ERR_INVALID_ARG;
    if (dx_ws_bytes(C_in, C_out, dtype, n, taps) == 0) return SV_ERR_UNSUPPORTED;
    if (n == 0) return SV_OK;
    return hip_status(launch_conv_bfrag(static_cast<const uint16_t*>(dY), N, static_cast<const uint16_t*>(P),
                                        nullptr, static_cast<uint16_t*>(dX), n, C_out, C_in, taps, stream));
}

namespace {

// Shared checks of the two phases of the weight gradient.
sv_status dw_phase_args(int64_t n, int32_t K, int32_t C_in, int32_t C_out, sv_dtype dtype, const void* workspace,
                        size_t workspace_bytes, DwPlan* plan) {
    int taps = 0;
    sv_status st = taps_of(K, &taps);
    if (st != SV_OK) return st;
    if ((st = conv_args_ok(n, taps, C_in, C_out, dtype, SV_KERNEL_AUTO)) != SV_OK) return st;
    *plan = plan_dw(n, C_in, C_out, dtype == SV_BF16, taps);
    const size_t need = dw_workspace_bytes(*plan);
    if (need > 0 && (!workspace || workspace_bytes < need)) return SV_ERR_WORKSPACE;
    if (workspace && reinterpret_cast<uintptr_t>(workspace) % 16) return SV_ERR_INVALID_ARG;
    return SV_OK;
}

}  // namespace

sv_status sv_sparseconv2d_bwd_dw_partials_k(const void* X, const int32_t* N, const void* dY, float* dW, float* db,
                                            int64_t n, int32_t K, int32_t C_in, int32_t C_out, sv_dtype dtype,
                                            int32_t accumulate, void* workspace, size_t workspace_bytes,
                                            hipStream_t stream) {
    DwPlan plan;
    sv_status st = dw_phase_args(n, K, C_in, C_out, dtype, workspace, workspace_bytes, &plan);
    if (st != SV_OK) return st;
    if (!dW || (n > 0 && (!X || !N || !dY))) return SV_ERR_INVALID_ARG;
    return hip_status(launch_dw_partials(plan, dtype == SV_BF16, X, N, dY, dW, db, n, C_in, C_out,
                                         accumulate ? 1 : 0, workspace, stream));
}

sv_status sv_sparseconv2d_bwd_dw_reduce_k(float* dW, float* db, int64_t n, int32_t K, int32_t C_in, int32_t C_out,
                                          sv_dtype dtype, int32_t accumulate, const void* workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
    DwPlan plan;
    sv_status st = dw_phase_args(n, K, C_in, C_out, dtype, workspace, workspace_bytes, &plan);
    if (st != SV_OK) return st;
    if (!dW) return SV_ERR_INVALID_ARG;
    return hip_status(launch_dw_reduce(plan, dW, db, C_in, C_out, accumulate ? 1 : 0, workspace, stream));
}

// ------------------------------------------------------------ chunk driver
namespace {

struct ChunkLayout {
    int K = 3, taps = 9;      // neighbourhood of the descriptor (ksize 0 reads as 3)
    int64_t max_tokens = 0;   // largest chunk, in tokens
    size_t n_bytes = 0;       // chunk-local N table
    size_t w_bytes = 0;       // forward weights repacked for the MFMA kernel
    size_t dw_bytes = 0;      // dW/db partials of the largest plan
    size_t n2_bytes = 0;      // second N table when dW runs on its own stream
    size_t p_bytes = 0;       // input-gradient weights in fragment order
    size_t total = 0;
    // the input-gradient weights sit after everything else
    size_t p_off() const { return n_bytes + w_bytes + dw_bytes + n2_bytes; }
};

int ksize_of(int32_t ksize) { return ksize == 0 ? 3 : ksize; }

// Upper bound of dw_workspace_bytes(plan_dw(toks, ...)) over toks <= max_tokens:
// a plan has at most 64 slices and, with more than one, at least 256 tokens
// per slice (both planners), so slices <= min(64, max_tokens / 256 + 1).
size_t dw_bytes_bound(int64_t max_tokens, int Ci, int Co, int taps) {
    const int64_t s = std::min<int64_t>(64, max_tokens / 256 + 1);
    const size_t part = s > 1 ? static_cast<size_t>(s) * taps * Ci * Co * sizeof(float) : 0;
    return align_up(part) + align_up(static_cast<size_t>(s) * Co * sizeof(float));
}

bool chunk_layout(const sv_chunked_desc* d, uint32_t passes, ChunkLayout* L) {
    if (!d || d->T < 0 || d->H <= 0 || d->W <= 0 ||
        d->chunk_frames <= 0 || d->C_in <= 0 || d->C_out <= 0 || !valid_dtype(d->dtype))
        return false;
    L->K = ksize_of(d->ksize);
    if (taps_of(L->K, &L->taps) != SV_OK) return false;
    const int32_t* ho = d->frame_offsets_host;
    if (!ho) {
        // No host copy of the offsets: the bound for chunks of chunk_frames
        // full frames (every chunk holds at most chunk_frames * H * W tokens).
        L->max_tokens = static_cast<int64_t>(std::min(d->T, d->chunk_frames)) * d->H * d->W;
        if (L->max_tokens > max_rows(L->taps)) return false;
        L->dw_bytes = (passes & SV_PASS_DW) ? dw_bytes_bound(L->max_tokens, d->C_in, d->C_out, L->taps) : 0;
    } else {
    if (ho[0] != 0) return false;
    for (int t = 0; t < d->T; ++t)
        if (ho[t + 1] < ho[t]) return false;
    L->max_tokens = 0;
    // With the dW pass even an empty video needs the (zero-token) plan's db partials.
    const bool bf = d->dtype == SV_BF16;
    L->dw_bytes = (passes & SV_PASS_DW)
                      ? dw_workspace_bytes(plan_dw(0, d->C_in, d->C_out, bf, L->taps))
                      : 0;
    for (int f0 = 0; f0 < d->T; f0 += d->chunk_frames) {
        const int f1 = std::min(d->T, f0 + d->chunk_frames);
        const int64_t toks = static_cast<int64_t>(ho[f1]) - ho[f0];
        L->max_tokens = std::max(L->max_tokens, toks);
        if (passes & SV_PASS_DW)
            L->dw_bytes = std::max(L->dw_bytes, dw_workspace_bytes(plan_dw(toks, d->C_in, d->C_out, bf, L->taps)));
    }
    }
    L->n_bytes = align_up(static_cast<size_t>(L->max_tokens) * L->taps * sizeof(int32_t));
    L->w_bytes = (passes & SV_PASS_FWD) ? fwd_ws_bytes(d->C_in, d->C_out, d->dtype, L->max_tokens, L->taps) : 0;
    const bool split = d->dw_stream && (passes & SV_PASS_DW) && (passes & (SV_PASS_FWD | SV_PASS_DX));
    L->n2_bytes = split ? L->n_bytes : 0;
    L->p_bytes = ((passes & SV_PASS_DX) && d->kernel != SV_KERNEL_VALU)
                     ? dx_ws_bytes(d->C_in, d->C_out, d->dtype, L->max_tokens, L->taps)
                     : 0;
    L->total = L->n_bytes + L->w_bytes + L->dw_bytes + L->n2_bytes + L->p_bytes;
    return true;
}

// Events of a call, destroyed when the call returns (a recorded event is
// released by the runtime once the device has passed it).  They only order
// kernels of this device on two streams, so they are made without the
// system-scope fence: a device-scope release suffices, and the fence's
// cache write-back held the next kernel on the recording stream for ~6 us.
struct CallEvents {
    hipEvent_t ev[6] = {};
    int made = 0;
    bool make(int k) {
        for (; made < k; ++made)
            if (hipEventCreateWithFlags(&ev[made], hipEventDisableTiming | hipEventDisableSystemFence) !=
                hipSuccess)
                return false;
        return true;
    }
    ~CallEvents() {
        for (int i = 0; i < made; ++i) (void)hipEventDestroy(ev[i]);
    }
};

}  // namespace

size_t sv_chunked_workspace_bytes(const sv_chunked_desc* desc, uint32_t passes) {
    ChunkLayout L;
    if (!chunk_layout(desc, passes, &L)) return 0;
    return L.total;
}

sv_status sv_sparseconv2d_chunked(const sv_chunked_desc* d, uint32_t passes, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    int taps0 = 0;
    if (d && taps_of(ksize_of(d->ksize), &taps0) == SV_ERR_UNSUPPORTED) return SV_ERR_UNSUPPORTED;
    ChunkLayout L;
    if (!chunk_layout(d, passes, &L)) return SV_ERR_INVALID_ARG;
    if (!d->frame_offsets_host) {
        // The chunk boundaries are needed on the host: copy the offsets and
        // wait for the copy (the one place the library waits on a stream).
        // The workspace was sized for the bound, which covers the exact
        // layout of the call below.
        if (!d->frame_offsets) return SV_ERR_INVALID_ARG;
        std::vector<int32_t> ho(static_cast<size_t>(d->T) + 1);
        if (hipMemcpyAsync(ho.data(), d->frame_offsets, ho.size() * sizeof(int32_t), hipMemcpyDeviceToHost,
                           stream) != hipSuccess ||
            hipStreamSynchronize(stream) != hipSuccess)
            return SV_ERR_HIP;
        sv_chunked_desc dd = *d;
        dd.frame_offsets_host = ho.data();
        ChunkLayout E;
        if (!chunk_layout(&dd, passes, &E)) return SV_ERR_INVALID_ARG;
        if (E.total > L.total) return SV_ERR_INVALID_ARG;    // offsets beyond full frames
        return sv_sparseconv2d_chunked(&dd, passes, workspace, workspace_bytes, stream);
    }
    if (passes & ~(SV_PASS_FWD | SV_PASS_DX | SV_PASS_DW)) return SV_ERR_INVALID_ARG;
    if (!valid_kernel(d->kernel)) return SV_ERR_INVALID_ARG;
    if (static_cast<int64_t>(d->H) * d->W > kMaxCells) return SV_ERR_UNSUPPORTED;
    const int64_t n = d->frame_offsets_host[d->T];
    if (n > max_rows(L.taps)) return SV_ERR_INVALID_ARG;
    if (!d->frame_offsets || (n > 0 && !d->coords)) return SV_ERR_INVALID_ARG;
    if ((passes & SV_PASS_FWD) && (!d->X || !d->Wt || !d->Y)) return SV_ERR_INVALID_ARG;
    if ((passes & SV_PASS_DX) && (!d->dY || !d->Wt || !d->dX)) return SV_ERR_INVALID_ARG;
    if ((passes & SV_PASS_DW) && (!d->X || !d->dY || !d->dW)) return SV_ERR_INVALID_ARG;
    bool m;
    // Every chunk holds at most L.max_tokens tokens: a kernel that fits the
    // largest chunk fits them all.
    if ((passes & SV_PASS_FWD) &&
        choose(d->kernel, d->dtype, false, d->C_in, d->C_out, L.max_tokens, L.taps, &m) != SV_OK)
        return SV_ERR_UNSUPPORTED;
    if ((passes & SV_PASS_DX) &&
        choose(d->kernel, d->dtype, true, d->C_in, d->C_out, L.max_tokens, L.taps, &m) != SV_OK)
        return SV_ERR_UNSUPPORTED;
    if (L.total > 0 && (!workspace || workspace_bytes < L.total)) return SV_ERR_WORKSPACE;
    if (workspace && reinterpret_cast<uintptr_t>(workspace) % 256) return SV_ERR_INVALID_ARG;

    const size_t es = d->dtype == SV_BF16 ? 2 : 4;
    int32_t* Nc = static_cast<int32_t*>(workspace);
    void* Vw = static_cast<char*>(workspace) + L.n_bytes;
    void* dws = static_cast<char*>(workspace) + L.n_bytes + L.w_bytes;
    bool fwd_mfma = false, dx_mfma = false;
    if (passes & SV_PASS_DX) choose(d->kernel, d->dtype, true, d->C_in, d->C_out, L.max_tokens, L.taps, &dx_mfma);
    void* Pw = (dx_mfma && L.p_bytes > 0 && reinterpret_cast<uintptr_t>(d->Wt) % 16 == 0)
                   ? static_cast<char*>(workspace) + L.p_off()
                   : nullptr;
    if (Pw && d->T > 0) {
        // the input gradient's weights, in fragment order, once for every chunk
        sv_status st = hip_status(launch_repack_frag(static_cast<const uint16_t*>(d->Wt), static_cast<uint16_t*>(Pw),
                                                     d->C_in, d->C_out, L.taps, true, stream));
        if (st != SV_OK) return st;
    }
    if (passes & SV_PASS_FWD) {
        choose(d->kernel, d->dtype, false, d->C_in, d->C_out, L.max_tokens, L.taps, &fwd_mfma);
        if (fwd_mfma && d->T > 0) {
            // the weights are repacked once for every chunk
            sv_status st = hip_status(launch_repack_fwd(static_cast<const uint16_t*>(d->Wt),
                                                        static_cast<uint16_t*>(Vw), d->C_in, d->C_out, L.taps,
                                                        stream));
            if (st != SV_OK) return st;
        }
    }
    const int32_t* ho = d->frame_offsets_host;
    // With a dW stream (the workspace then has a second N table): chunk c's
    // table is built into table c & 1 on `stream`; the dW stream waits for
    // that build (ev_idx), and the build of chunk c + 2 into the same table
    // waits for chunk c's dW (ev_dw).
    const bool split = L.n2_bytes > 0 && d->dw_stream != stream;
    hipStream_t ds = split ? d->dw_stream : stream;
    int32_t* Ntab[2] = {Nc, split ? reinterpret_cast<int32_t*>(static_cast<char*>(dws) + L.dw_bytes) : Nc};
    CallEvents E;
    hipEvent_t ev_start = nullptr, ev_join = nullptr, *ev_idx = nullptr, *ev_dw = nullptr;
    if (split && d->T > 0) {
        if (!E.make(6)) return SV_ERR_HIP;
        ev_start = E.ev[0];
        ev_idx = E.ev + 1;
        ev_dw = E.ev + 3;
        ev_join = E.ev[5];
        if (hipEventRecord(ev_start, stream) != hipSuccess || hipStreamWaitEvent(ds, ev_start, 0) != hipSuccess)
            return SV_ERR_HIP;
    }
    bool first = true;
    for (int f0 = 0, ci = 0; f0 < d->T; f0 += d->chunk_frames, ++ci) {
        const int f1 = std::min(d->T, f0 + d->chunk_frames);
        const int64_t t0 = ho[f0], nc = static_cast<int64_t>(ho[f1]) - t0;
        int32_t* Nc = Ntab[ci & 1];
        if (split && ci >= 2 && hipStreamWaitEvent(stream, ev_dw[ci & 1], 0) != hipSuccess) return SV_ERR_HIP;
        sv_status st = hip_status(launch_build_index(d->coords, d->frame_offsets, f0, f1 - f0, d->H, d->W, L.K,
                                                     nc, t0, Nc, nullptr, d->err_flag, stream));
        if (st != SV_OK) return st;
        if (split && hipEventRecord(ev_idx[ci & 1], stream) != hipSuccess) return SV_ERR_HIP;
        const char* X = d->X ? static_cast<const char*>(d->X) + t0 * d->C_in * es : nullptr;
        const char* dY = d->dY ? static_cast<const char*>(d->dY) + t0 * d->C_out * es : nullptr;
        char* Yc = (passes & SV_PASS_FWD) ? static_cast<char*>(d->Y) + t0 * d->C_out * es : nullptr;
        char* dXc = (passes & SV_PASS_DX) ? static_cast<char*>(d->dX) + t0 * d->C_in * es : nullptr;
        if (fwd_mfma && dx_mfma) {
            // With the weight gradients on their own stream the paired
            // launch takes about half the chip (larger tiles): a dW
            // workgroup needs more LDS than a conv workgroup leaves free on
            // its compute unit, so with the conv grid on every unit the
            // chunk's dW waited for it (config 4: 0.506-0.517 -> 0.490-0.492
            // ms per pass).
            st = run_fwd_dx_pair(X, dY, Nc, d->Wt, Vw, Pw, d->bias, Yc, dXc, nc, d->C_in, d->C_out, L.taps,
                                 split ? kBfragSlots / 2 : kBfragSlots, stream);
            if (st != SV_OK) return st;
        } else {
            if (passes & SV_PASS_FWD) {
                st = run_fwd_prepared(fwd_mfma, X, Nc, d->Wt, Vw, d->bias, Yc, nc, d->C_in, d->C_out, L.taps,
                                      d->dtype, stream);
                if (st != SV_OK) return st;
            }
            if (passes & SV_PASS_DX) {
                st = run_dx(dY, Nc, d->Wt, dXc, nc, d->C_in, d->C_out, L.taps, d->dtype, d->kernel, stream, nullptr,
                            Pw);
                if (st != SV_OK) return st;
            }
        }
        if (passes & SV_PASS_DW) {
            if (split && hipStreamWaitEvent(ds, ev_idx[ci & 1], 0) != hipSuccess) return SV_ERR_HIP;
            const DwPlan plan = plan_dw(nc, d->C_in, d->C_out, d->dtype == SV_BF16, L.taps);
            st = hip_status(launch_dw(plan, d->dtype == SV_BF16, X, Nc, dY, d->dW, d->db, nc, d->C_in,
                                      d->C_out, first ? 0 : 1, dws, ds));
            if (st != SV_OK) return st;
            if (split && hipEventRecord(ev_dw[ci & 1], ds) != hipSuccess) return SV_ERR_HIP;
        }
        first = false;
    }
    if (split && d->T > 0 &&
        (hipEventRecord(ev_join, ds) != hipSuccess || hipStreamWaitEvent(stream, ev_join, 0) != hipSuccess))
        return SV_ERR_HIP;
    if (first && (passes & SV_PASS_DW)) {
        // No frames at all: the gradients of an empty sum are zero.
        const DwPlan plan = plan_dw(0, d->C_in, d->C_out, d->dtype == SV_BF16, L.taps);
        return hip_status(launch_dw(plan, d->dtype == SV_BF16, d->X, Nc, d->dY, d->dW, d->db, 0, d->C_in,
                                    d->C_out, 0, dws, stream));
    }
    return sync_check(d->err_flag, stream);
}

// ------------------------------------------------- host-streamed chunk driver
}  // extern "C"

namespace {

constexpr int kSets = 4;              // staging sets of the host-streamed driver
constexpr int kAhead = 2;             // chunks uploaded ahead of the compute

struct HostLayout {
    ChunkLayout dev;                  // N table, repacked weights, dW partials
    int max_frames = 0;
    size_t coords_b = 0, offs_b = 0, x_b = 0, dy_b = 0, y_b = 0, dx_b = 0;
    size_t set_bytes = 0;             // one staging set
    size_t total = 0;
};

bool host_layout(const sv_chunked_host_desc* d, uint32_t passes, HostLayout* L) {
    if (!d || !d->frame_offsets_host) return false;
    // The device driver's layout reads only host fields; build it from a
    // descriptor carrying the same ones.
    sv_chunked_desc dd{};
    dd.T = d->T; dd.H = d->H; dd.W = d->W; dd.C_in = d->C_in; dd.C_out = d->C_out;
    dd.dtype = d->dtype; dd.kernel = d->kernel; dd.chunk_frames = d->chunk_frames; dd.ksize = d->ksize;
    dd.frame_offsets_host = d->frame_offsets_host;
    if (!chunk_layout(&dd, passes, &L->dev)) return false;
    const size_t es = d->dtype == SV_BF16 ? 2 : 4;
    const size_t tok = static_cast<size_t>(L->dev.max_tokens);
    L->max_frames = std::min(d->chunk_frames, std::max(d->T, 0));
    L->coords_b = align_up(tok * sizeof(int32_t));
    L->offs_b = align_up((static_cast<size_t>(L->max_frames) + 1) * sizeof(int32_t));
    L->x_b = (passes & (SV_PASS_FWD | SV_PASS_DW)) ? align_up(tok * d->C_in * es) : 0;
    L->dy_b = (passes & (SV_PASS_DX | SV_PASS_DW)) ? align_up(tok * d->C_out * es) : 0;
    L->y_b = (passes & SV_PASS_FWD) ? align_up(tok * d->C_out * es) : 0;
    L->dx_b = (passes & SV_PASS_DX) ? align_up(tok * d->C_in * es) : 0;
    L->set_bytes = L->coords_b + L->offs_b + L->x_b + L->dy_b + L->y_b + L->dx_b;
    L->total = L->dev.total + kSets * L->set_bytes;
    return true;
}

struct Staging {
    int32_t* coords;
    int32_t* offs;
    char *X, *dY, *Y, *dX;
};

}  // namespace

extern "C" {

size_t sv_chunked_host_workspace_bytes(const sv_chunked_host_desc* desc, uint32_t passes) {
    HostLayout L;
    if (passes & ~(SV_PASS_FWD | SV_PASS_DX | SV_PASS_DW)) return 0;
    if (!host_layout(desc, passes, &L)) return 0;
    return L.total;
}

sv_status sv_sparseconv2d_chunked_host(const sv_chunked_host_desc* d, uint32_t passes, void* workspace,
                                       size_t workspace_bytes, hipStream_t compute, hipStream_t h2d,
                                       hipStream_t d2h) {
    int taps0 = 0;
    if (d && taps_of(ksize_of(d->ksize), &taps0) == SV_ERR_UNSUPPORTED) return SV_ERR_UNSUPPORTED;
    HostLayout L;
    if (passes & ~(SV_PASS_FWD | SV_PASS_DX | SV_PASS_DW)) return SV_ERR_INVALID_ARG;
    if (!host_layout(d, passes, &L)) return SV_ERR_INVALID_ARG;
    if (!valid_kernel(d->kernel)) return SV_ERR_INVALID_ARG;
    if (compute == h2d || compute == d2h || h2d == d2h) return SV_ERR_INVALID_ARG;
    if (static_cast<int64_t>(d->H) * d->W > kMaxCells) return SV_ERR_UNSUPPORTED;
    const int32_t* ho = d->frame_offsets_host;
    const int64_t n = ho[d->T];
    const int taps = L.dev.taps;
    if (n > max_rows(taps)) return SV_ERR_INVALID_ARG;
    if (n > 0 && !d->coords_host) return SV_ERR_INVALID_ARG;
    if ((passes & SV_PASS_FWD) && (!d->X_host || !d->Wt || !d->Y_host)) return SV_ERR_INVALID_ARG;
    if ((passes & SV_PASS_DX) && (!d->dY_host || !d->Wt || !d->dX_host)) return SV_ERR_INVALID_ARG;
    if ((passes & SV_PASS_DW) && (!d->X_host || !d->dY_host || !d->dW)) return SV_ERR_INVALID_ARG;
    bool m;
    if ((passes & SV_PASS_FWD) &&
        choose(d->kernel, d->dtype, false, d->C_in, d->C_out, L.dev.max_tokens, taps, &m) != SV_OK)
        return SV_ERR_UNSUPPORTED;
    if ((passes & SV_PASS_DX) &&
        choose(d->kernel, d->dtype, true, d->C_in, d->C_out, L.dev.max_tokens, taps, &m) != SV_OK)
        return SV_ERR_UNSUPPORTED;
    if (L.total > 0 && (!workspace || workspace_bytes < L.total)) return SV_ERR_WORKSPACE;
    if (workspace && reinterpret_cast<uintptr_t>(workspace) % 256) return SV_ERR_INVALID_ARG;

    // The host arrays must be page-locked (the copy engines then move them
    // without staging and the copies are asynchronous); anything else is an
    // argument error.
    auto pinned = [](const void* h) {
        void* p = nullptr;
        return !h || hipHostGetDevicePointer(&p, const_cast<void*>(h), 0) == hipSuccess;
    };
    if (!pinned(d->coords_host) || !pinned(d->frame_offsets_host) ||
        !pinned((passes & (SV_PASS_FWD | SV_PASS_DW)) ? d->X_host : nullptr) ||
        !pinned((passes & (SV_PASS_DX | SV_PASS_DW)) ? d->dY_host : nullptr) ||
        !pinned((passes & SV_PASS_FWD) ? d->Y_host : nullptr) || !pinned((passes & SV_PASS_DX) ? d->dX_host : nullptr)) {
        (void)hipGetLastError();          // clear the query's error state
        return SV_ERR_INVALID_ARG;
    }

    // Workspace: N table | repacked weights | dW partials | staging sets.
    const size_t es = d->dtype == SV_BF16 ? 2 : 4;
    char* base = static_cast<char*>(workspace);
    int32_t* Nc = reinterpret_cast<int32_t*>(base);
    void* Vw = base + L.dev.n_bytes;
    void* dws = base + L.dev.n_bytes + L.dev.w_bytes;
    Staging st[kSets];
    for (int b = 0; b < kSets; ++b) {
        char* p = base + L.dev.total + b * L.set_bytes;
        st[b].coords = reinterpret_cast<int32_t*>(p);
        p += L.coords_b;
        st[b].offs = reinterpret_cast<int32_t*>(p);
        p += L.offs_b;
        st[b].X = p;  p += L.x_b;
        st[b].dY = p; p += L.dy_b;
        st[b].Y = p;  p += L.y_b;
        st[b].dX = p;
    }

    bool fwd_mfma = false, dx_mfma = false;
    if (passes & SV_PASS_DX) choose(d->kernel, d->dtype, true, d->C_in, d->C_out, L.dev.max_tokens, taps, &dx_mfma);
    void* Pw = (dx_mfma && L.dev.p_bytes > 0 && reinterpret_cast<uintptr_t>(d->Wt) % 16 == 0)
                   ? base + L.dev.p_off()
                   : nullptr;
    if (Pw && d->T > 0) {
        sv_status st0 = hip_status(launch_repack_frag(static_cast<const uint16_t*>(d->Wt), static_cast<uint16_t*>(Pw),
                                                      d->C_in, d->C_out, taps, true, compute));
        if (st0 != SV_OK) return st0;
    }
    if (passes & SV_PASS_FWD) {
        choose(d->kernel, d->dtype, false, d->C_in, d->C_out, L.dev.max_tokens, taps, &fwd_mfma);
        if (fwd_mfma && d->T > 0) {
            sv_status st0 = hip_status(launch_repack_fwd(static_cast<const uint16_t*>(d->Wt),
                                                         static_cast<uint16_t*>(Vw), d->C_in, d->C_out, taps,
                                                         compute));
            if (st0 != SV_OK) return st0;
        }
    }
    const int nchunks = d->T > 0 ? (d->T + d->chunk_frames - 1) / d->chunk_frames : 0;
    if (nchunks == 0) {
        if (!(passes & SV_PASS_DW)) return SV_OK;
        // No frames at all: the gradients of an empty sum are zero.
        const DwPlan plan = plan_dw(0, d->C_in, d->C_out, d->dtype == SV_BF16, taps);
        return hip_status(launch_dw(plan, d->dtype == SV_BF16, nullptr, Nc, nullptr, d->dW, d->db, 0, d->C_in,
                                    d->C_out, 0, dws, compute));
    }

    // Chunk c uses staging set c % kSets.  ev_in[b]: the chunk's inputs are
    // in set b; ev_done[b]: its compute finished; ev_out[b]: its results left
    // set b (set b is free again).  The transfers are copy-engine copies
    // (hipMemcpyAsync), and neither copy stream ever waits on another
    // stream's event: a copy queued behind such a wait that has not fired
    // holds the host thread in the runtime until it fires, which put the
    // whole pipeline in lockstep.  The host orders them instead: it queues
    // chunk c's download once its compute has finished, and the upload into
    // a set once that set's previous chunk has been downloaded.  With uploads
    // kAhead = 2 chunks ahead of the compute and four sets, each of those
    // waits is for work queued about a chunk earlier, so that the host keeps
    // the copy engines and the compute stream fed.  The compute stream waits
    // on the upload stream's events on the GPU (kernels only).
    hipEvent_t ev[3 * kSets + 1] = {};
    for (int i = 0; i < 3 * kSets + 1; ++i)
        if (hipEventCreateWithFlags(&ev[i], hipEventDisableTiming) != hipSuccess) {
            for (int k = 0; k < i; ++k) (void)hipEventDestroy(ev[k]);
            return SV_ERR_HIP;
        }
    hipEvent_t* ev_in = ev;
    hipEvent_t* ev_done = ev + kSets;
    hipEvent_t* ev_out = ev + 2 * kSets;
    hipEvent_t ev_start = ev[3 * kSets];
    auto chunk_bounds = [&](int ci, int* f0, int* f1, int64_t* t0, int64_t* nc) {
        *f0 = ci * d->chunk_frames;
        *f1 = std::min(d->T, *f0 + d->chunk_frames);
        *t0 = ho[*f0];
        *nc = static_cast<int64_t>(ho[*f1]) - *t0;
    };
    auto h2d_copy = [&](void* dst, const void* src, int64_t bytes) {
        return bytes > 0 ? hipMemcpyAsync(dst, src, static_cast<size_t>(bytes), hipMemcpyHostToDevice, h2d)
                         : hipSuccess;
    };
    auto d2h_copy = [&](void* dst, const void* src, int64_t bytes) {
        return bytes > 0 ? hipMemcpyAsync(dst, src, static_cast<size_t>(bytes), hipMemcpyDeviceToHost, d2h)
                         : hipSuccess;
    };
    auto upload = [&](int ci) -> hipError_t {
        const int b = ci % kSets;
        int f0, f1;
        int64_t t0, nc;
        chunk_bounds(ci, &f0, &f1, &t0, &nc);
        hipError_t e = hipSuccess;
        if (ci >= kSets && (e = hipEventSynchronize(ev_out[b])) != hipSuccess) return e;
        if ((e = h2d_copy(st[b].coords, d->coords_host + t0, nc * static_cast<int64_t>(sizeof(int32_t)))))
            return e;
        if ((e = h2d_copy(st[b].offs, ho + f0, (f1 - f0 + 1) * static_cast<int64_t>(sizeof(int32_t))))) return e;
        if (L.x_b && (e = h2d_copy(st[b].X, static_cast<const char*>(d->X_host) + t0 * d->C_in * es,
                                   nc * d->C_in * static_cast<int64_t>(es))))
            return e;
        if (L.dy_b && (e = h2d_copy(st[b].dY, static_cast<const char*>(d->dY_host) + t0 * d->C_out * es,
                                    nc * d->C_out * static_cast<int64_t>(es))))
            return e;
        return hipEventRecord(ev_in[b], h2d);
    };
    auto download = [&](int ci) -> hipError_t {
        const int b = ci % kSets;
        int f0, f1;
        int64_t t0, nc;
        chunk_bounds(ci, &f0, &f1, &t0, &nc);
        hipError_t e = hipEventSynchronize(ev_done[b]);
        if (e != hipSuccess) return e;
        if ((passes & SV_PASS_FWD) && (e = d2h_copy(static_cast<char*>(d->Y_host) + t0 * d->C_out * es, st[b].Y,
                                                    nc * d->C_out * static_cast<int64_t>(es))))
            return e;
        if ((passes & SV_PASS_DX) && (e = d2h_copy(static_cast<char*>(d->dX_host) + t0 * d->C_in * es, st[b].dX,
                                                   nc * d->C_in * static_cast<int64_t>(es))))
            return e;
        return hipEventRecord(ev_out[b], d2h);
    };
    auto compute_chunk = [&](int ci) -> sv_status {
        const int b = ci % kSets;
        int f0, f1;
        int64_t t0, nc;
        chunk_bounds(ci, &f0, &f1, &t0, &nc);
        if (hipStreamWaitEvent(compute, ev_in[b], 0) != hipSuccess) return SV_ERR_HIP;
        // The staged slices hold global frame offsets and the chunk's own
        // coordinates; the index kernel reads offs[f0 + f] and coords[k]
        // for global k, so it gets both bases shifted back.
        const int32_t* coords_g = st[b].coords - t0;
        const int32_t* offs_g = st[b].offs - f0;
        sv_status s2 = hip_status(launch_build_index(coords_g, offs_g, f0, f1 - f0, d->H, d->W, L.dev.K, nc, t0,
                                                     Nc, nullptr, d->err_flag, compute));
        if (s2 != SV_OK) return s2;
        if (fwd_mfma && dx_mfma) {
            s2 = run_fwd_dx_pair(st[b].X, st[b].dY, Nc, d->Wt, Vw, Pw, d->bias, st[b].Y, st[b].dX, nc, d->C_in,
                                 d->C_out, taps, kBfragSlots, compute);
            if (s2 != SV_OK) return s2;
        } else {
            if (passes & SV_PASS_FWD) {
                s2 = run_fwd_prepared(fwd_mfma, st[b].X, Nc, d->Wt, Vw, d->bias, st[b].Y, nc, d->C_in, d->C_out,
                                      taps, d->dtype, compute);
                if (s2 != SV_OK) return s2;
            }
            if (passes & SV_PASS_DX) {
                s2 = run_dx(st[b].dY, Nc, d->Wt, st[b].dX, nc, d->C_in, d->C_out, taps, d->dtype, d->kernel,
                            compute, nullptr, Pw);
                if (s2 != SV_OK) return s2;
            }
        }
        if (passes & SV_PASS_DW) {
            const DwPlan plan = plan_dw(nc, d->C_in, d->C_out, d->dtype == SV_BF16, taps);
            s2 = hip_status(launch_dw(plan, d->dtype == SV_BF16, st[b].X, Nc, st[b].dY, d->dW, d->db, nc, d->C_in,
                                      d->C_out, ci == 0 ? 0 : 1, dws, compute));
            if (s2 != SV_OK) return s2;
        }
        return hip_status(hipEventRecord(ev_done[b], compute));
    };
    auto run = [&]() -> sv_status {
        // The staging sets are free once everything enqueued on `compute`
        // before this call is done (a previous call on this workspace ends
        // there, after its last copies).
        if (hipEventRecord(ev_start, compute) != hipSuccess || hipEventSynchronize(ev_start) != hipSuccess)
            return SV_ERR_HIP;
        for (int ci = 0; ci < std::min(nchunks, kAhead); ++ci)
            if (upload(ci) != hipSuccess) return SV_ERR_HIP;
        for (int ci = 0; ci < nchunks; ++ci) {
            const sv_status s2 = compute_chunk(ci);
            if (s2 != SV_OK) return s2;
            if (ci >= 1 && download(ci - 1) != hipSuccess) return SV_ERR_HIP;
            if (ci + kAhead < nchunks && upload(ci + kAhead) != hipSuccess) return SV_ERR_HIP;
        }
        if (download(nchunks - 1) != hipSuccess) return SV_ERR_HIP;
        // Synchronising `compute` then covers every copy of the call.
        return hip_status(hipStreamWaitEvent(compute, ev_out[(nchunks - 1) % kSets], 0));
    };
    const sv_status result = run();
    for (int i = 0; i < 3 * kSets + 1; ++i) (void)hipEventDestroy(ev[i]);
    return result != SV_OK ? result : sync_check(d->err_flag, compute);
}

// ------------------------------------------------------ bottleneck adapter
namespace {

// Workspace of the adapter: the identity table of the two projections, then
// either the shared repack region of the three forwards or dH2 | dH1 | the
// shared dW region of the three weight gradients (the passes run in order
// on one stream, so one region serves them all).
struct AdapterLayout {
    int taps = 0;
    size_t id_bytes = 0, h_bytes = 0, rest_bytes = 0, p_bytes = 0, total = 0;
};

sv_status adapter_layout(bool backward, int64_t n, int32_t K, int32_t C, int32_t r, sv_dtype dt, AdapterLayout* L) {
    sv_status st = taps_of(K, &L->taps);
    if (st != SV_OK) return st;
    if (n < 0 || n > max_rows(L->taps) || C <= 0 || r <= 0 || !valid_dtype(dt)) return SV_ERR_INVALID_ARG;
    const size_t es = dt == SV_BF16 ? 2 : 4;
    L->id_bytes = align_up(static_cast<size_t>(n) * sizeof(int32_t));
    if (!backward) {
        L->h_bytes = 0;
        L->rest_bytes = std::max({fwd_ws_bytes(C, r, dt, n, 1), fwd_ws_bytes(r, r, dt, n, L->taps),
                                  fwd_ws_bytes(r, C, dt, n, 1), dense_res_ws_bytes(r, C)});
    } else {
        L->h_bytes = align_up(static_cast<size_t>(n) * r * es);
        const bool bf = dt == SV_BF16;
        L->rest_bytes = std::max({dw_workspace_bytes(plan_dw(n, r, C, bf, 1)),
                                  dw_workspace_bytes(plan_dw(n, r, r, bf, L->taps)),
                                  dw_workspace_bytes(plan_dw(n, C, r, bf, 1))});
        // the input gradients' weights in fragment order, where the fragment
        // kernel takes them (the last one, with its residual, never does)
        L->p_bytes = std::max({dx_ws_bytes(r, C, dt, n, 1), dx_ws_bytes(r, r, dt, n, L->taps),
                               dense_res_ws_bytes(r, C)});
    }
    L->total = L->id_bytes + 2 * L->h_bytes + align_up(L->rest_bytes) + align_up(L->p_bytes);
    return SV_OK;
}

// One forward pass of a layer (repack into `V` when the MFMA kernel runs).
sv_status adapter_layer_fwd(const void* X, const int32_t* N, const void* Wt, const void* bias, const void* R,
                            void* Y, int64_t n, int32_t Ci, int32_t Co, int taps, sv_dtype dt, sv_kernel kernel,
                            void* V, hipStream_t s) {
    bool mfma = false;
    sv_status st = choose(kernel, dt, false, Ci, Co, n, taps, &mfma);
    if (st != SV_OK) return st;
    if (mfma && R && taps == 1 && dense_res_supported(dt == SV_BF16, Ci, Co, n)) {
        // the up-projection with its residual: the dense streaming kernel
        st = hip_status(launch_repack_dense(static_cast<const uint16_t*>(Wt), static_cast<uint16_t*>(V), Ci, Co,
                                            false, s));
        if (st != SV_OK || n == 0) return st;
        return hip_status(launch_dense_res(static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(V),
                                           static_cast<const uint16_t*>(bias), static_cast<const uint16_t*>(R),
                                           static_cast<uint16_t*>(Y), n, Ci, Co, s));
    }
    if (mfma) {
        // with a residual the layer runs on k_conv_mfma: its per-tap layout
        st = hip_status(launch_repack_fwd(static_cast<const uint16_t*>(Wt), static_cast<uint16_t*>(V), Ci, Co,
                                          taps, s, R == nullptr));
        if (st != SV_OK) return st;
    }
    return run_fwd_prepared(mfma, X, N, Wt, V, bias, Y, n, Ci, Co, taps, dt, s, R);
}

}  // namespace

size_t sv_adapter_workspace_bytes(int32_t backward, int64_t n, int32_t K, int32_t C, int32_t r, sv_dtype dtype) {
    AdapterLayout L;
    if (adapter_layout(backward != 0, n, K, C, r, dtype, &L) != SV_OK) return 0;
    return L.total;
}

sv_status sv_adapter_fwd(const void* X, const int32_t* N, int64_t n, int32_t K, int32_t C, int32_t r,
                         const void* Wd, const void* bd, const void* Wc, const void* bc, const void* Wu,
                         const void* bu, void* H1, void* H2, void* Y, sv_dtype dtype, sv_kernel kernel,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
    AdapterLayout L;
    sv_status st = adapter_layout(false, n, K, C, r, dtype, &L);
    if (st != SV_OK) return st;
    if (!valid_kernel(kernel)) return SV_ERR_INVALID_ARG;
    if (!Wd || !Wc || !Wu || (n > 0 && (!X || !N || !H1 || !H2 || !Y))) return SV_ERR_INVALID_ARG;
    bool m;
    // every pass must fit the requested kernel before anything is enqueued
    if (choose(kernel, dtype, false, C, r, n, 1, &m) != SV_OK ||
        choose(kernel, dtype, false, r, r, n, L.taps, &m) != SV_OK ||
        choose(kernel, dtype, false, r, C, n, 1, &m) != SV_OK)
        return SV_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < L.total) return SV_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 256) return SV_ERR_INVALID_ARG;
    if (n == 0) return SV_OK;
    int32_t* I = static_cast<int32_t*>(workspace);
    void* V = static_cast<char*>(workspace) + L.id_bytes;
    if ((st = hip_status(launch_iota(I, n, stream))) != SV_OK) return st;
    if ((st = adapter_layer_fwd(X, I, Wd, bd, nullptr, H1, n, C, r, 1, dtype, kernel, V, stream)) != SV_OK)
        return st;
    if ((st = adapter_layer_fwd(H1, N, Wc, bc, nullptr, H2, n, r, r, L.taps, dtype, kernel, V, stream)) != SV_OK)
        return st;
    return adapter_layer_fwd(H2, I, Wu, bu, X, Y, n, r, C, 1, dtype, kernel, V, stream);
}

sv_status sv_adapter_bwd(const void* X, const int32_t* N, int64_t n, int32_t K, int32_t C, int32_t r,
                         const void* Wd, const void* Wc, const void* Wu, const void* H1, const void* H2,
                         const void* dY, void* dX, float* dWd, float* dbd, float* dWc, float* dbc, float* dWu,
                         float* dbu, sv_dtype dtype, sv_kernel kernel, void* workspace, size_t workspace_bytes,
                         hipStream_t stream, hipStream_t dw_stream) {
    AdapterLayout L;
    sv_status st = adapter_layout(true, n, K, C, r, dtype, &L);
    if (st != SV_OK) return st;
    if (!valid_kernel(kernel)) return SV_ERR_INVALID_ARG;
    if (!Wd || !Wc || !Wu || !dWd || !dWc || !dWu) return SV_ERR_INVALID_ARG;
    if (n > 0 && (!X || !N || !H1 || !H2 || !dY || !dX)) return SV_ERR_INVALID_ARG;
    bool m;
    if (choose(kernel, dtype, true, r, C, n, 1, &m) != SV_OK ||
        choose(kernel, dtype, true, r, r, n, L.taps, &m) != SV_OK ||
        choose(kernel, dtype, true, C, r, n, 1, &m) != SV_OK)
        return SV_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < L.total) return SV_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 256) return SV_ERR_INVALID_ARG;
    const bool bf = dtype == SV_BF16;
    char* base = static_cast<char*>(workspace);
    int32_t* I = reinterpret_cast<int32_t*>(base);
    void* dH2 = base + L.id_bytes;
    void* dH1 = base + L.id_bytes + L.h_bytes;
    void* dws = base + L.id_bytes + 2 * L.h_bytes;
    void* Pw = L.p_bytes ? base + L.id_bytes + 2 * L.h_bytes + align_up(L.rest_bytes) : nullptr;
    // An input gradient on the fragment kernel where it takes the shape: its
    // weights repacked into Pw first (the calls run in order on `stream`, so
    // one region serves all three).
    auto dx_layer = [&](const void* g, const int32_t* Nt, const void* Wt, void* out, int32_t Ci, int32_t Co,
                        int taps, const void* R) -> sv_status {
        if (R && Pw && taps == 1 && kernel != SV_KERNEL_VALU && dense_res_supported(bf, Co, Ci, n)) {
            // dX = R + g W^T on the dense streaming kernel (K = Co contracted,
            // Ci produced), when the MFMA path takes the layer
            bool m = false;
            const sv_status s0 = choose(kernel, dtype, true, Ci, Co, n, taps, &m);
            if (s0 != SV_OK) return s0;
            if (m) {
                const sv_status s1 = hip_status(launch_repack_dense(static_cast<const uint16_t*>(Wt),
                                                                    static_cast<uint16_t*>(Pw), Co, Ci, true, stream));
                if (s1 != SV_OK || n == 0) return s1;
                return hip_status(launch_dense_res(static_cast<const uint16_t*>(g), static_cast<const uint16_t*>(Pw),
                                                   nullptr, static_cast<const uint16_t*>(R),
                                                   static_cast<uint16_t*>(out), n, Co, Ci, stream));
            }
        }
        const void* P = nullptr;
        if (Pw && !R && kernel != SV_KERNEL_VALU && dx_ws_bytes(Ci, Co, dtype, n, taps) > 0 &&
            reinterpret_cast<uintptr_t>(Wt) % 16 == 0) {
            const sv_status s1 = hip_status(launch_repack_frag(static_cast<const uint16_t*>(Wt),
                                                               static_cast<uint16_t*>(Pw), Ci, Co, taps, true,
                                                               stream));
            if (s1 != SV_OK) return s1;
            P = Pw;
        }
        return run_dx(g, Nt, Wt, out, n, Ci, Co, taps, dtype, kernel, stream, R, P);
    };
    // With a dW stream each weight gradient waits (event) for the tensor it
    // reads, produced on `stream`; they run in order on that stream and share
    // one partials region.  Nothing either stream reads is overwritten.
    const bool split = dw_stream && dw_stream != stream && n > 0;
    hipStream_t ds = split ? dw_stream : stream;
    CallEvents E;
    if (split && !E.make(4)) return SV_ERR_HIP;
    auto handoff = [&](int e) -> sv_status {
        if (!split) return SV_OK;
        if (hipEventRecord(E.ev[e], stream) != hipSuccess || hipStreamWaitEvent(ds, E.ev[e], 0) != hipSuccess)
            return SV_ERR_HIP;
        return SV_OK;
    };
    if ((st = hip_status(launch_iota(I, n, stream))) != SV_OK) return st;
    if ((st = handoff(0)) != SV_OK) return st;
    // up-projection: dWu, dbu, then dH2 = dY Wu^T
    if ((st = hip_status(launch_dw(plan_dw(n, r, C, bf, 1), bf, H2, I, dY, dWu, dbu, n, r, C, 0, dws, ds))) !=
        SV_OK)
        return st;
    if ((st = dx_layer(dY, I, Wu, dH2, r, C, 1, nullptr)) != SV_OK) return st;
    if ((st = handoff(1)) != SV_OK) return st;
    // K x K convolution: dWc, dbc, then dH1
    if ((st = hip_status(launch_dw(plan_dw(n, r, r, bf, L.taps), bf, H1, N, dH2, dWc, dbc, n, r, r, 0, dws,
                                   ds))) != SV_OK)
        return st;
    if ((st = dx_layer(dH2, N, Wc, dH1, r, r, L.taps, nullptr)) != SV_OK) return st;
    if ((st = handoff(2)) != SV_OK) return st;
    // down-projection: dWd, dbd, then dX = dY + dH1 Wd^T
    if ((st = hip_status(launch_dw(plan_dw(n, C, r, bf, 1), bf, X, I, dH1, dWd, dbd, n, C, r, 0, dws, ds))) !=
        SV_OK)
        return st;
    if ((st = dx_layer(dH1, I, Wd, dX, C, r, 1, dY)) != SV_OK) return st;
    if (split && (hipEventRecord(E.ev[3], ds) != hipSuccess || hipStreamWaitEvent(stream, E.ev[3], 0) != hipSuccess))
        return SV_ERR_HIP;
    return SV_OK;
}

// ------------------------------------------------------ cross-attention
namespace {

bool a16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

sv_status xattn_args_ok(int64_t m, int64_t n, int32_t d, sv_dtype dtype) {
    if (m < 0 || n < 0 || m > 65535 || !valid_dtype(dtype)) return SV_ERR_INVALID_ARG;
    if (!xattn_supported(d)) return SV_ERR_UNSUPPORTED;
    return SV_OK;
}

float xattn_scale(float scale, int32_t d) { return scale == 0.f ? 1.f / sqrtf(static_cast<float>(d)) : scale; }

}  // namespace

size_t sv_xattn_workspace_bytes(int32_t backward, int64_t m, int64_t n, int32_t d) {
    if (m < 0 || n < 0 || !xattn_supported(d)) return 0;
    const XattnPlan p = plan_xattn(m, n, d);
    return backward ? p.bwd_bytes : p.fwd_bytes;
}

sv_status sv_xattn_fwd(const void* Q, const void* X, int64_t m, int64_t n, int32_t d, float scale, sv_dtype dtype,
                       void* O, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    sv_status st = xattn_args_ok(m, n, d, dtype);
    if (st != SV_OK) return st;
    if (m == 0) return SV_OK;
    if (!Q || !O || !lse || (n > 0 && !X) || !std::isfinite(scale)) return SV_ERR_INVALID_ARG;
    if (!a16(Q) || !a16(O) || (n > 0 && !a16(X))) return SV_ERR_INVALID_ARG;
    const XattnPlan p = plan_xattn(m, n, d);
    if (!workspace || workspace_bytes < p.fwd_bytes) return SV_ERR_WORKSPACE;
    if (!a16(workspace)) return SV_ERR_INVALID_ARG;
    return hip_status(launch_xattn_fwd(p, dtype == SV_BF16, Q, X, static_cast<int>(m), n, d, xattn_scale(scale, d), O,
                                       lse, workspace, stream));
}

sv_status sv_xattn_bwd(const void* Q, const void* X, const void* O, const void* dO, const float* lse, int64_t m,
                       int64_t n, int32_t d, float scale, sv_dtype dtype, float* dQ, void* dX, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
    sv_status st = xattn_args_ok(m, n, d, dtype);
    if (st != SV_OK) return st;
    if (m == 0) {
        // no queries: nothing flows back into the keys
        if (n == 0) return SV_OK;
        if (!dX) return SV_ERR_INVALID_ARG;
        return hip_status(launch_stage_scatter(nullptr, nullptr, 0, dX, n, d, dtype == SV_BF16 ? 2 : 4, stream));
    }
    if (!Q || !O || !dO || !lse || !dQ || (n > 0 && (!X || !dX)) || !std::isfinite(scale)) return SV_ERR_INVALID_ARG;
    if (!a16(Q) || !a16(O) || !a16(dO) || !a16(dQ) || (n > 0 && (!a16(X) || !a16(dX)))) return SV_ERR_INVALID_ARG;
    const XattnPlan p = plan_xattn(m, n, d);
    if (p.bwd_bytes > 0 && (!workspace || workspace_bytes < p.bwd_bytes)) return SV_ERR_WORKSPACE;
    if (workspace && !a16(workspace)) return SV_ERR_INVALID_ARG;
    return hip_status(launch_xattn_bwd(p, dtype == SV_BF16, Q, X, O, dO, lse, static_cast<int>(m), n, d,
                                       xattn_scale(scale, d), dQ, dX, workspace, stream));
}

sv_status sv_stage_gather(const void* src, int64_t n_src, const int32_t* rows, int64_t n_rows, void* dst,
                          int32_t C, sv_dtype dtype, hipStream_t stream) {
    if (n_src < 0 || n_rows < 0 || C <= 0 || !valid_dtype(dtype)) return SV_ERR_INVALID_ARG;
    if (n_rows > 0 && (!src || !rows || !dst)) return SV_ERR_INVALID_ARG;
    return hip_status(launch_stage_gather(src, n_src, rows, n_rows, dst, C, dtype == SV_BF16 ? 2 : 4, stream));
}

sv_status sv_stage_scatter(const void* src, const int32_t* rows, int64_t n_rows, void* dst, int64_t n_dst,
                           int32_t C, sv_dtype dtype, hipStream_t stream) {
    if (n_dst < 0 || n_rows < 0 || C <= 0 || !valid_dtype(dtype)) return SV_ERR_INVALID_ARG;
    if (n_dst > 0 && !dst) return SV_ERR_INVALID_ARG;
    if (n_rows > 0 && (!src || !rows)) return SV_ERR_INVALID_ARG;
    return hip_status(launch_stage_scatter(src, rows, n_rows, dst, n_dst, C, dtype == SV_BF16 ? 2 : 4, stream));
}

const char* sv_status_string(sv_status s) {
    switch (s) {
        case SV_OK: return "SV_OK";
        case SV_ERR_INVALID_ARG: return "SV_ERR_INVALID_ARG: invalid argument";
        case SV_ERR_UNSUPPORTED: return "SV_ERR_UNSUPPORTED: shape or dtype not supported by the kernel";
        case SV_ERR_WORKSPACE: return "SV_ERR_WORKSPACE: workspace missing or too small";
        case SV_ERR_HIP: return "SV_ERR_HIP: a HIP call failed";
        case SV_ERR_COORD_RANGE: return "SV_ERR_COORD_RANGE: coordinate outside the grid";
        case SV_ERR_DUPLICATE_COORD: return "SV_ERR_DUPLICATE_COORD: two tokens on one grid cell";
    }
    return "unknown sv_status";
}

const char* sv_version(void) { return "svconv 0.1.0 gfx950"; }

}  // extern "C"
