// noalloc.hip -- moe_ffn_forward_noalloc: the layer with its workspace in a
// file-scope device array of the library instead of caller memory, for callers
// that cannot allocate device memory.
//
// The array is one per device (each GPU the library runs on holds its own copy
// until the process ends).  In host code its name is only a stand-in for the
// symbol, not a device address: the first call on a device, with that device
// current, asks the runtime for the address of that device's copy and keeps it;
// every use from the host (the kernels' workspace pointer) goes through that
// address.  The forward's kernels write every workspace byte they read within
// the call, so the array needs no clearing between calls.
#include <mutex>

#include "internal.h"

namespace {

constexpr size_t kScratchBytes = MOE_FFN_NOALLOC_WORKSPACE_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

extern "C" moe_ffn_status moe_ffn_forward_noalloc(moe_ffn_plan_t plan, const moe_ffn_tensors *tensors,
                                                  int32_t n_tokens, hipStream_t stream) {
    if (!plan || !tensors) return moeffn::set_error(MOE_FFN_ERR_INVALID_ARG, "plan and tensors must not be NULL");
    if (plan->L.total > kScratchBytes)
        return moeffn::set_error(MOE_FFN_ERR_WORKSPACE_TOO_SMALL,
                                 "the plan needs " + std::to_string(plan->L.total) +
                                     " bytes of workspace; the library's static workspace holds " +
                                     std::to_string(kScratchBytes) + " (plan fewer max_tokens)");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return moeffn::set_error(MOE_FFN_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (dev != plan->d.device)
        return moeffn::set_error(MOE_FFN_ERR_WRONG_DEVICE, "current device differs from desc.device");
    if (dev < 0 || dev >= kMaxDevices)
        return moeffn::set_error(MOE_FFN_ERR_UNSUPPORTED, "device ordinal beyond the static workspace table");
    void *ws = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (!g_scratch_ptr[dev]) {
            void *p = nullptr;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // this device's copy (it is current)
            if (e != hipSuccess || !p)
                return moeffn::set_error(MOE_FFN_ERR_HIP, std::string("hipGetSymbolAddress: ") +
                                                             hipGetErrorString(e));
            g_scratch_ptr[dev] = p;
        }
        ws = g_scratch_ptr[dev];
    }
    return moe_ffn_forward(plan, tensors, n_tokens, ws, kScratchBytes, stream);
}
