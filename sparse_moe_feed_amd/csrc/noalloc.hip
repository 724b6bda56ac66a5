// noalloc.hip -- moe_forward for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the workspace is a static device array of the library instead
// of a caller buffer.
//
// `scratch` is a file-scope __device__ array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code the array's name only stands in for the symbol, so its device address
// on the current GPU is looked up once per device with hipGetSymbolAddress and
// kept; only that address is ever handed to kernels.  The kernels are those
// of moe_forward, which already treats its workspace as uninitialised
// scratch (everything that must start at zero is cleared by its own
// launches), so the contents the previous call left behind do no harm.
#include "moe.h"
#include "moe_kernels.h"

#include <mutex>

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current GPU (looked up on the first
// call on that GPU).  Returns MOE_ERR_HIP with the HIP error text on failure.
moe_status scratch_on_current_device(void **out) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) {
        moe::set_last_error(hipGetErrorString(err));
        return MOE_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        moe::set_last_error("moe_forward_noalloc: device ordinal beyond the library's table");
        return MOE_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess || !ptr) {
            moe::set_last_error(err != hipSuccess ? hipGetErrorString(err)
                                                  : "hipGetSymbolAddress gave no address");
            return MOE_ERR_HIP;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_forward_noalloc(const moe_desc *desc, int64_t T, const void *x,
                                          const void *w_router, const float *router_bias,
                                          const void *w_gate_up, const void *w_down,
                                          const void *w_sh_gate_up, const void *w_sh_down,
                                          const void *sh_gate, float *out, int32_t *topk_idx,
                                          float *topk_w, void *stream) {
    moe_status st = moe::check_forward_args(desc, T, x, w_router, router_bias, w_gate_up, w_down,
                                            w_sh_gate_up, w_sh_down, sh_gate, out, topk_idx,
                                            topk_w);
    if (st != MOE_OK) return st;
    moe_workspace_layout lay;
    st = moe_workspace_query(desc, T, &lay);
    if (st != MOE_OK) return st;
    if (lay.total > kScratchBytes) {
        moe::set_last_error("moe_forward_noalloc: the call needs more workspace than the "
                            "library's static scratch (MOE_NOALLOC_SCRATCH_BYTES)");
        return MOE_ERR_WORKSPACE;
    }
    if (T == 0) return MOE_OK;
    void *ws = nullptr;
    st = scratch_on_current_device(&ws);
    if (st != MOE_OK) return st;
    return moe_forward(desc, T, x, w_router, router_bias, w_gate_up, w_down, w_sh_gate_up,
                       w_sh_down, sh_gate, out, topk_idx, topk_w, ws, kScratchBytes, stream);
}
