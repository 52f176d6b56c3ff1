// Allocation-free form of the weight-gradient call, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The split-K partials that
// sv_sparseconv2d_bwd_dw_k keeps in the caller's workspace live here in a
// file-scope device array instead; everything else -- the plan, the kernels,
// the summation order -- is the workspace call's, so the two give the same
// bits.
#include <limits>
#include <mutex>

#include "internal.h"

using namespace svc;

// One copy per device, held from module load until the process ends.  In
// host code `scratch` is only a stand-in for the symbol: its device address
// comes from hipGetSymbolAddress, per device, and only that address is ever
// handed to a kernel.
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = SV_NOALLOC_SCRATCH_BYTES;

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's scratch address, looked up on the first call on that
// device (with that device current) and cached.
sv_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SV_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return SV_OK;
}

}  // namespace

extern "C" {

sv_status sv_sparseconv2d_bwd_dw_noalloc_k(const void* X, const int32_t* N, const void* dY, float* dW, float* db,
                                           int64_t n, int32_t K, int32_t C_in, int32_t C_out, sv_dtype dtype,
                                           int32_t accumulate, hipStream_t stream) {
    if (K < 1 || K % 2 == 0) return SV_ERR_INVALID_ARG;
    if (K > 7) return SV_ERR_UNSUPPORTED;
    const int taps = K * K;
    if (n < 0 || n > std::numeric_limits<int32_t>::max() / taps || C_in <= 0 || C_out <= 0) return SV_ERR_INVALID_ARG;
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_INVALID_ARG;
    if (!dW || (n > 0 && (!X || !N || !dY))) return SV_ERR_INVALID_ARG;
    const DwPlan plan = plan_dw(n, C_in, C_out, dtype == SV_BF16, taps);
    if (dw_workspace_bytes(plan) > kScratchBytes) return SV_ERR_WORKSPACE;
    void* ws = nullptr;
    const sv_status st = scratch_address(&ws);
    if (st != SV_OK) return st;
    return launch_dw(plan, dtype == SV_BF16, X, N, dY, dW, db, n, C_in, C_out, accumulate ? 1 : 0, ws, stream) ==
                   hipSuccess
               ? SV_OK
               : SV_ERR_HIP;
}

}  // extern "C"
