// moe_static.hip -- moe_layer_forward_static: the MoE layer forward ("MoE 路由与专家流式加载"
// §1) for callers that cannot allocate device memory.  Its scratch is `scratch`, a
// file-scope device array of MOE_STATIC_SCRATCH_BYTES that the library's code object
// carries, instead of a caller workspace.
//
// In host code the name `scratch` is a host-side stand-in, not a device address.  The
// device address of each GPU's copy is looked up once per device, with that device
// current, by hipGetSymbolAddress and kept per device; only that address is ever
// passed to a kernel.  The call then runs the same validation and launch sequence as
// moe_layer_forward with the array as its workspace.  Nothing is allocated and
// nothing needs clearing (the workspace contents on entry are ignored by every
// kernel); overlapping calls on one GPU race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe.h"
#include "moe_internal.h"

namespace moe {

static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kStaticMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kStaticMaxDevices];  // device address of `scratch` on each device
}  // namespace

// This device's copy of `scratch` (the current device, dev), or nullptr if the lookup
// failed.  Looked up once per device.
static void *scratch_on(int dev) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace moe

using namespace moe;

extern "C" int moe_layer_forward_static(const moe_layer *L, const float *x, int32_t T, void *out,
                                        int32_t out_dtype, const moe_route_out *dbg, void *stream) {
    int rc;
    if ((rc = layer_forward_validate(L, x, T, out, out_dtype))) return rc;
    if (T == 0) return MOE_OK;
    const size_t need = moe_workspace_bytes(L, T);
    if (need == 0) return MOE_EINVAL;
    if (need > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_EWORKSPACE;
    if ((rc = device_ok())) return rc;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kStaticMaxDevices) {
        (void)hipGetLastError();
        return MOE_EDEVICE;
    }
    void *ws = scratch_on(dev);
    if (!ws) return MOE_EDEVICE;
    return layer_forward_run(L, x, T, out, out_dtype, dbg, ws, (hipStream_t)stream, nullptr);
}
