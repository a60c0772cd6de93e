// ss1_mlp_forward_static: the SS1 MLP pair with its h workspace in a static
// device array instead of a caller buffer, for callers that cannot allocate.
//
// The array is a file-scope device variable.  In host code its name is only a
// host-side stand-in, not a device address, so the first call on each device
// looks the address up with hipGetSymbolAddress (with that device current)
// and keeps it per device; kernels only ever receive that pointer.  Every GPU
// the library runs on holds its own copy until the process ends.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <mutex>

#include "ss1_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[SS1_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (nullptr on failure).
void* scratch_address() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" ss1_status ss1_mlp_forward_static(const ss1_tensor* x, const ss1_layer* up, const ss1_layer* down,
                                             ss1_tensor* y, void* stream) {
    if (!x || !up || !down || !y) return SS1_ERR_NULL;
    if (x->dtype != SS1_BF16 && x->dtype != SS1_F32) return SS1_ERR_DTYPE;
    const int64_t N1 = up->W_c.rows;
    const int64_t e = x->dtype == SS1_BF16 ? 2 : 4;
    if (N1 <= 0 || N1 > static_cast<int64_t>(SS1_STATIC_SCRATCH_BYTES) / e) return SS1_ERR_SHAPE;
    int64_t R = static_cast<int64_t>(SS1_STATIC_SCRATCH_BYTES) / (N1 * e);
    if (R >= 256) R -= R % 256;
    ss1_tensor h{nullptr, x->dtype, 0, R, N1};
    if (x->rows == 0) return ss1::mlp_forward_ws(x, up, down, &h, y, stream);  // checks only
    h.data = scratch_address();
    if (!h.data) return SS1_ERR_HIP;
    return ss1::mlp_forward_ws(x, up, down, &h, y, stream);
}
