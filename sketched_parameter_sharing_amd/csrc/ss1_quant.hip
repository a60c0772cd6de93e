// Per-row fp8 quantization of a compressed weight: the SS1 summary page's
// "Measured effects" apply post-training quantization on top of SS1 models
// and its "Limitations" note that quantized SS1 kernels were not built.  Here
// each row n of W_c gets one float32 scale, scale[n] = max_k |W_c[n][k]| / 448
// (IEEE division; 1 for an all-zero row), and each entry the OCP E4M3 code
// nearest to W_c[n][k] / scale[n] (ties to even).  448 is E4M3's largest
// finite value, so the quotient never leaves the format's range (the clamp
// below only absorbs the last bit of the float32 division).
//
// One block of 256 threads per row: a max-reduction over the row, then the
// conversion of pairs with v_cvt_pk_fp8_f32.  A one-time setup step, like
// the plan.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "ss1_device.h"
#include "ss1_internal.h"

namespace ss1 {

namespace {

__device__ __forceinline__ float load_f(const uint16_t* p, size_t i) { return __uint_as_float(uint32_t(p[i]) << 16); }
__device__ __forceinline__ float load_f(const float* p, size_t i) { return p[i]; }

template <typename T>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const T* __restrict__ W, uint8_t* __restrict__ Q,
                                                           float* __restrict__ scale, int Kc) {
    __shared__ float red[4];
    const int n = blockIdx.x;
    const size_t base = static_cast<size_t>(n) * Kc;
    float amax = 0.0f;
    for (int k = threadIdx.x; k < Kc; k += 256) amax = fmaxf(amax, fabsf(load_f(W, base + k)));
    // wave maximum, then across the four waves
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float sc = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    if (threadIdx.x == 0) scale[n] = sc;
    // Kc is even (a multiple of the chunk width): convert pairs
    for (int k = 2 * threadIdx.x; k < Kc; k += 512) {
        const float a = fminf(fmaxf(__fdiv_rn(load_f(W, base + k), sc), -448.0f), 448.0f);
        const float b = fminf(fmaxf(__fdiv_rn(load_f(W, base + k + 1), sc), -448.0f), 448.0f);
        const uint32_t packed = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false));
        *reinterpret_cast<uint16_t*>(Q + base + k) = static_cast<uint16_t>(packed & 0xFFFFu);
    }
}

}  // namespace

ss1_status launch_quantize_fp8(const void* W, int32_t dtype, int64_t N, int64_t Kc, void* Q, float* scale,
                               void* stream) {
    if (N == 0) return SS1_OK;
    if (dtype == SS1_BF16)
        hipLaunchKernelGGL((quantize_fp8_kernel<uint16_t>), dim3(static_cast<unsigned>(N)), dim3(256), 0,
                           static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(W),
                           static_cast<uint8_t*>(Q), scale, static_cast<int>(Kc));
    else
        hipLaunchKernelGGL((quantize_fp8_kernel<float>), dim3(static_cast<unsigned>(N)), dim3(256), 0,
                           static_cast<hipStream_t>(stream), static_cast<const float*>(W),
                           static_cast<uint8_t*>(Q), scale, static_cast<int>(Kc));
    return hipGetLastError() == hipSuccess ? SS1_OK : SS1_ERR_HIP;
}

}  // namespace ss1
