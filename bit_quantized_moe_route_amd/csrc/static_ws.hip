// moe_layer_forward_static: moe_layer_forward with its workspace in a
// file-scope device array instead of a caller's buffer, for callers that
// cannot allocate device memory (code under HIP graph capture, serving loops
// that must not allocate).
//
// The array is one per GPU (each device that loads the library's code object
// holds its own copy, until the process ends).  Host code never passes the
// array's name to a kernel: its device address is looked up once per device
// with hipGetSymbolAddress (with that device current) and kept; the
// workspace pointer handed to moe_layer_forward is that address.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "internal.h"

namespace moeq {
namespace {

__device__ __align__(256) uint8_t scratch[MOE_STATIC_WS_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];   // device address of `scratch`, per device
std::mutex g_scratch_mu;

// The current device's address of the array (looked up on the first call on
// that device); NULL with the error recorded on failure.
void* scratch_ptr(int* status) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *status = fail(MOE_EHIP, std::string("moe_layer_forward_static: hipGetDevice: ") +
                                     hipGetErrorString(e));
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *status = fail(MOE_EINVAL, "moe_layer_forward_static: device index beyond 63");
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *status = fail(MOE_EHIP, std::string("moe_layer_forward_static: hipGetSymbolAddress: ") +
                                         hipGetErrorString(e));
            return nullptr;
        }
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace
}  // namespace moeq

using namespace moeq;

extern "C" int moe_layer_forward_static(const moe_qlayer* layer, const uint16_t* x_bf16,
                                        const float* logits, int64_t T, int32_t k,
                                        const float* y_shared, int32_t* topk_ids, float* topk_w,
                                        float* out, void* stream) {
    set_error("");
    if (!layer) return fail(MOE_EINVAL, "moe_layer_forward_static: layer is NULL");
    const size_t need = moe_layer_forward_workspace_bytes(layer, T, k);
    if (need > (size_t)MOE_STATIC_WS_BYTES)
        return fail(MOE_EWORKSPACE, "moe_layer_forward_static: this batch needs " +
                                        std::to_string(need) +
                                        " bytes of workspace; the static workspace holds " +
                                        std::to_string((size_t)MOE_STATIC_WS_BYTES) +
                                        " (use moe_layer_forward with a caller's buffer)");
    int status = MOE_OK;
    void* ws = scratch_ptr(&status);
    if (!ws) return status;
    return moe_layer_forward(layer, x_bf16, logits, T, k, y_shared, topk_ids, topk_w, out, ws,
                             (size_t)MOE_STATIC_WS_BYTES, stream);
}
