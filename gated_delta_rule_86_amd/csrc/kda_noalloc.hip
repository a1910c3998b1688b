// kda_noalloc.hip -- kda_fwd_noalloc: the forward pass for callers that cannot allocate
// device memory (code under stream capture, tight serving loops, harnesses that forbid
// hipMalloc).  Same kernels as kda_fwd_ex; the workspace is a static device array of this
// file, one copy per GPU, held until the process ends.
#include <mutex>

#include <hip/hip_runtime.h>

#include "kda.h"
#include "kda_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)KDA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % kda::kAlign == 0, "scratch size");

// The workspace of kda_fwd_noalloc.  In host code `scratch` names a host-side stand-in,
// not device memory: only the per-device address from hipGetSymbolAddress is ever passed on.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// Device address of `scratch` on `dev`, resolved once per device with that device current.
void *scratch_on(int dev)
{
    if (dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::call_once(g_once[dev], [dev]() {
        int cur = -1;
        g_err[dev] = hipGetDevice(&cur);
        if (g_err[dev] != hipSuccess)
            return;
        if (cur != dev && (g_err[dev] = hipSetDevice(dev)) != hipSuccess)
            return;
        void *p = nullptr;
        g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
        if (cur != dev) {
            const hipError_t e = hipSetDevice(cur);
            if (g_err[dev] == hipSuccess)
                g_err[dev] = e;
        }
    });
    return g_err[dev] == hipSuccess ? g_ptr[dev] : nullptr;
}

}  // namespace

extern "C" kda_status kda_fwd_noalloc(const void *q, const void *k, const void *v, const void *g,
                                      const void *beta, float scale, void *out, const float *A_log,
                                      const float *dt_bias, float lower_bound, const void *initial_state,
                                      kda_state_dtype initial_state_dtype, void *final_state,
                                      kda_state_dtype final_state_dtype, const int64_t *cu_seqlens,
                                      const int64_t *cu_seqlens_host, int64_t B, int64_t T, int64_t H,
                                      int64_t N, int64_t K, int64_t V, void *stream, uint32_t flags)
{
    // sizes first, before any HIP call: a problem whose workspace exceeds the static array
    // is rejected (invalid sizes give 0 here and are reported by the full validation below)
    const size_t need = kda_fwd_workspace_size(B, T, H, cu_seqlens ? N : (N == B ? B : 0), cu_seqlens != nullptr);
    if (need > kScratchBytes)
        return KDA_ERR_SCRATCH;
    int dev = -1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess)
        return KDA_ERR_HIP;
    void *ws = scratch_on(dev);
    if (!ws)
        return KDA_ERR_HIP;
    // every table the kernels read from the workspace is written earlier in the same call
    // (the chunk table first, then the segment states in pass A and the scan), so nothing
    // needs clearing between calls
    return kda_fwd_ex(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                      initial_state_dtype, final_state, final_state_dtype, cu_seqlens, cu_seqlens_host, B,
                      T, H, N, K, V, ws, kScratchBytes, stream, flags);
}
