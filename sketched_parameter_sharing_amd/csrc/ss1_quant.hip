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
// conversion of pairs with v_cvt_pk_fp8_f32.  For weights a one-time setup
// step, like the plan; the fp8 layer (ss1_forward_fp8) also quantizes its
// input rows this way on every call, where rows of a multiple of 8 elements
// take 16-byte loads, stay in registers between the two passes and leave as
// 8-byte stores.
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

// Eight consecutive values of a row as float32 (16-byte bf16 or 2 x 16-byte
// float32 loads).
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
    const uint4 r = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// The same quantization for rows of Kc % 8 == 0 (every layer's weight and
// input rows here): each thread takes 8-element vectors tid, tid + 256, ...,
// keeps up to VR of them in registers between the max-reduction and the
// conversion (rows up to 2048*VR elements are read once), and stores each
// vector's 8 codes with one 8-byte store.  Codes and scale are those of
// quantize_fp8_kernel.
template <typename T, int VR>
__global__ __launch_bounds__(256) void quantize_fp8_vec_kernel(const T* __restrict__ W, uint8_t* __restrict__ Q,
                                                               float* __restrict__ scale, int Kc) {
    __shared__ float red[4];
    const int n = blockIdx.x;
    const size_t base = static_cast<size_t>(n) * Kc;
    const int nv = Kc / 8;
    float keep[VR][8];
    float amax = 0.0f;
#pragma unroll
    for (int r = 0; r < VR; ++r) {
        const int v = threadIdx.x + r * 256;
        if (v < nv) {
            load8(W + base + 8 * static_cast<size_t>(v), keep[r]);
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(keep[r][i]));
        }
    }
    for (int v = threadIdx.x + VR * 256; v < nv; v += 256) {
        float t[8];
        load8(W + base + 8 * static_cast<size_t>(v), t);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(t[i]));
    }
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float sc = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    if (threadIdx.x == 0) scale[n] = sc;
    auto convert = [&](const float (&t)[8], int v) {
        uint32_t w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float a0 = fminf(fmaxf(__fdiv_rn(t[4 * h], sc), -448.0f), 448.0f);
            const float a1 = fminf(fmaxf(__fdiv_rn(t[4 * h + 1], sc), -448.0f), 448.0f);
            const float a2 = fminf(fmaxf(__fdiv_rn(t[4 * h + 2], sc), -448.0f), 448.0f);
            const float a3 = fminf(fmaxf(__fdiv_rn(t[4 * h + 3], sc), -448.0f), 448.0f);
            const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
            w[h] = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, lo, true));
        }
        *reinterpret_cast<uint2*>(Q + base + 8 * static_cast<size_t>(v)) = make_uint2(w[0], w[1]);
    };
#pragma unroll
    for (int r = 0; r < VR; ++r) {
        const int v = threadIdx.x + r * 256;
        if (v < nv) convert(keep[r], v);
    }
    for (int v = threadIdx.x + VR * 256; v < nv; v += 256) {
        float t[8];
        load8(W + base + 8 * static_cast<size_t>(v), t);
        convert(t, v);
    }
}

}  // namespace

ss1_status launch_quantize_fp8(const void* W, int32_t dtype, int64_t N, int64_t Kc, void* Q, float* scale,
                               void* stream) {
    if (N == 0) return SS1_OK;
    if (Kc % 8 == 0) {
        if (dtype == SS1_BF16)
            hipLaunchKernelGGL((quantize_fp8_vec_kernel<uint16_t, 8>), dim3(static_cast<unsigned>(N)), dim3(256), 0,
                               static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(W),
                               static_cast<uint8_t*>(Q), scale, static_cast<int>(Kc));
        else
            hipLaunchKernelGGL((quantize_fp8_vec_kernel<float, 8>), dim3(static_cast<unsigned>(N)), dim3(256), 0,
                               static_cast<hipStream_t>(stream), static_cast<const float*>(W),
                               static_cast<uint8_t*>(Q), scale, static_cast<int>(Kc));
        return hipGetLastError() == hipSuccess ? SS1_OK : SS1_ERR_HIP;
    }
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
