// csa_attention_noalloc: the fused CSA step without a caller workspace, for
// callers that cannot allocate device memory.  Its work area is a file-scope
// device array of kScratchBytes, one copy per GPU the library runs on, held
// until the process ends.  Host code never passes the array's name to a kernel
// (on the host that name is only a stand-in): the first call on a device takes
// the array's device address with hipGetSymbolAddress, with that device
// current, and keeps it per device.  Nothing in the work area has to start at
// zero (every part the kernels read back is written earlier in the same call),
// so no call clears it.  Calls that overlap on one GPU share the array and race.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "api_internal.hpp"

namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the device the call runs on (the current one).
csa_status scratch_address(void *stream, void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return csa_api::fail(CSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (stream != nullptr) {
        hipDevice_t sdev = 0;
        e = hipStreamGetDevice((hipStream_t)stream, &sdev);
        if (e != hipSuccess) return csa_api::fail(CSA_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
        if ((int)sdev != dev)
            return csa_api::fail(CSA_ERR_UNSUPPORTED, "the stream belongs to device %d but device %d is current",
                                 (int)sdev, dev);
    }
    if (dev < 0 || dev >= kMaxDevices)
        return csa_api::fail(CSA_ERR_UNSUPPORTED, "device %d: the static work area is tracked for devices 0..%d", dev,
                             kMaxDevices - 1);
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || p == nullptr)
                return csa_api::fail(CSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                                     hipGetErrorString(e));
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return CSA_OK;
}

}  // namespace

extern "C" csa_status csa_attention_noalloc(const csa_dims *d, const void *q, const void *q_idx, const float *w,
                                            const void *const *k_idx, const void *const *kv, const void *const *v,
                                            const void *const *win, const void *const *win_v,
                                            const int32_t *win_pos0, const int32_t *win_rows,
                                            const int32_t *seq_len, const int32_t *q_pos, const float *sink,
                                            float *out, float *lse, int32_t *topk_idx_out, float *scores_out,
                                            void *stream) {
    size_t need = 0;
    csa_status s = csa_workspace_size(d, CSA_OP_ATTENTION, &need);
    if (s != CSA_OK) return s;
    if (need > kScratchBytes)
        return csa_api::fail(CSA_ERR_WORKSPACE,
                             "csa_attention_noalloc: these sizes need %zu bytes of work area, the static one holds "
                             "%zu (use csa_attention with a caller workspace)",
                             need, kScratchBytes);
    void *ws = nullptr;
    if ((s = scratch_address(stream, &ws)) != CSA_OK) return s;
    return csa_api::attention_impl(d, q, q_idx, w, k_idx, kv, v, win, win_v, win_pos0, win_rows, seq_len, q_pos,
                                   sink, out, lse, topk_idx_out, scores_out, ws, kScratchBytes, stream);
}
