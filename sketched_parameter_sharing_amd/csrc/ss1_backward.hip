// Backward of the SS1 forward (the SS1 summary page, "Limitations": the
// backward pass is not reduced).  With y[:, g-block] = z_g W_c[g-block]^T:
//   dW_c[g-block] = dy[:, g-block]^T z_g                    (dw_kernel)
//   dx[:, j-chunk] = sum_g sign[g][j] (dy[:, g-block] W_c[g-block])[:, hash[g][j]-chunk]
//                  = dy times the dense expansion of W_c          (dx_kernel)
// Both run on 16x16x32 bf16 MFMA with float32 accumulation; the operand whose
// rows run along the reduction dimension is staged transposed through LDS.
//
// dw_kernel: block = 4 waves, output tile 32 neurons (inside one group) x 128
//   compressed columns, wave w owning columns [32w, 32w+32).  Per chunk of 64
//   tokens the block writes dy^T [32][64] and the sketch z^T [128][64] into
//   LDS (the sketch summed in float32 over the c sources in ascending order
//   and rounded to bf16, as in the forward), then each wave runs 2 x 2 blocks x
//   2 k-steps of MFMA.  Tokens past M are zero.
// dx_kernel: block = 4 waves, output tile 128 tokens x 32 columns of one input
//   chunk j, wave w owning tokens [32w, 32w+32).  Per 32-neuron slice of each
//   group the block stages the W_c slice of compressed chunk hash[g][j],
//   transposed and with sign[g][j] on its sign bits, in LDS; dy is read
//   straight into the MFMA operand (its rows are contiguous along n).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "ss1_device.h"
#include "ss1_internal.h"

namespace ss1 {

namespace {

using namespace dev;

constexpr int kDwN = 32;    // neurons per dw block
constexpr int kDwK = 128;   // compressed columns per dw block
constexpr int kDwM = 64;    // tokens per LDS chunk
constexpr int kDwP = kDwM + 8;  // LDS pitch (elements)

template <int C_T>
__global__ __launch_bounds__(256) void dw_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ dy,
                                                 const int32_t* __restrict__ pi, const int8_t* __restrict__ ps,
                                                 uint16_t* __restrict__ dw, int M, int K, int N, int J, int Jc,
                                                 int c_rt, int BK, int BN) {
    __shared__ __align__(16) uint16_t dyT[kDwN * kDwP];
    __shared__ __align__(16) uint16_t zT[kDwK * kDwP];
    extern __shared__ uint32_t smem[];
    uint32_t* s_src = smem;
    int* s_cnt = reinterpret_cast<int*>(smem + J);

    const int c = (C_T > 0) ? C_T : c_rt;
    const int Kc = Jc * BK;
    const int tiles_per_group = BN / kDwN;
    const int g = blockIdx.x / tiles_per_group;
    const int n0 = g * BN + (blockIdx.x % tiles_per_group) * kDwN;
    const int k0 = blockIdx.y * kDwK;
    stage_plan<true>(pi, ps, g, J, Jc, c, BK, s_src, s_cnt);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int fr = lane & 15;
    const int fk = (lane >> 4) * 8;

    f32x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    for (int m0 = 0; m0 < M; m0 += kDwM) {
        // dy^T: thread -> token m0 + tid%64, neurons n0 + 8*(tid/64) .. +7
        {
            const int mm = tid & 63;
            const int n8 = (tid >> 6) * 8;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (m0 + mm < M) v = *reinterpret_cast<const uint4*>(dy + static_cast<size_t>(m0 + mm) * N + n0 + n8);
            const uint32_t e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dyT[(n8 + 2 * i) * kDwP + mm] = static_cast<uint16_t>(e[i] & 0xFFFFu);
                dyT[(n8 + 2 * i + 1) * kDwP + mm] = static_cast<uint16_t>(e[i] >> 16);
            }
        }
        // z^T: vector v -> token m0 + v%64, columns k0 + 8*(v/64) .. +7
#pragma unroll
        for (int i = 0; i < (kDwM * kDwK / 8) / 256; ++i) {
            const int v = tid + i * 256;
            const int mm = v & 63;
            const int kk = (v >> 6) * 8;
            const int kp = k0 + kk;
            uint4 packed = make_uint4(0, 0, 0, 0);
            if (m0 + mm < M && kp < Kc) {
                const int t = kp / BK;
                const int u = kp - t * BK;
                const uint16_t* xr = x + static_cast<size_t>(m0 + mm) * K + u;
                float s[8];
                for (int r = 0; r < c; ++r) {
                    const uint32_t e = s_src[t * c + r];
                    const uint4 raw = *reinterpret_cast<const uint4*>(xr + (e & kOffMask));
                    acc_sign8(s, raw, entry_sign(e), entry_sign_xor(e), r == 0);
                }
                packed = pack_bf16x8(s);
            }
            const uint32_t e[4] = {packed.x, packed.y, packed.z, packed.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                zT[(kk + 2 * q) * kDwP + mm] = static_cast<uint16_t>(e[q] & 0xFFFFu);
                zT[(kk + 2 * q + 1) * kDwP + mm] = static_cast<uint16_t>(e[q] >> 16);
            }
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < kDwM; ks += 32) {
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int a = 0; a < 2; ++a)
                af[a] = *reinterpret_cast<const bf16x8*>(dyT + (16 * a + fr) * kDwP + ks + fk);
#pragma unroll
            for (int b = 0; b < 2; ++b)
                bfr[b] = *reinterpret_cast<const bf16x8*>(zT + (wave * 32 + 16 * b + fr) * kDwP + ks + fk);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
        }
        __syncthreads();
    }
    // lane holds rows 4*(lane/16) + 0..3 and column lane%16 of each 16x16 block
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int col = k0 + wave * 32 + 16 * b + fr;
            if (col >= Kc) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + 16 * a + (lane >> 4) * 4 + q;
                dw[static_cast<size_t>(n) * Kc + col] = to_bf16_bits(acc[a][b][q]);
            }
        }
}

constexpr int kDxM = 128;   // tokens per dx block
constexpr int kDxU = 32;    // columns per dx block (inside one input chunk)
constexpr int kDxP = 32 + 8;  // LDS pitch of W^T (elements)

__global__ __launch_bounds__(256) void dx_kernel(const uint16_t* __restrict__ dy, const uint16_t* __restrict__ w,
                                                 const int32_t* __restrict__ pi, const int8_t* __restrict__ ps,
                                                 uint16_t* __restrict__ dx, int M, int K, int N, int J, int Jc,
                                                 int BK, int BN) {
    __shared__ __align__(16) uint16_t wT[kDxU * kDxP];
    const int Kc = Jc * BK;
    const int G = N / BN;
    const int m0 = blockIdx.x * kDxM;
    const int col0 = blockIdx.y * kDxU;   // dx columns [col0, col0 + 32)
    const int j = col0 / BK;
    const int uoff = col0 - j * BK;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int fr = lane & 15;
    const int fk = (lane >> 4) * 8;
    // this lane's two dy rows (MFMA A rows), clamped inside M (rows past M are never stored)
    const uint16_t* dyr[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int m = min(m0 + wave * 32 + 16 * a + fr, M - 1);
        dyr[a] = dy + static_cast<size_t>(m) * N + fk;
    }
    // W^T staging: thread t < 128 -> neuron t/4 of the slice, columns 8*(t%4) .. +7
    const int wn = tid >> 2;
    const int wu = (tid & 3) * 8;

    f32x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    for (int g = 0; g < G; ++g) {
        const int t = pi[static_cast<size_t>(g) * J + j];
        const uint32_t flip = ps[static_cast<size_t>(g) * J + j] < 0 ? 0x80008000u : 0u;
        const size_t wcol = static_cast<size_t>(t) * BK + uoff;
        for (int nn = 0; nn < BN; nn += 32) {
            const int nb = g * BN + nn;
            if (tid < 128) {
                const uint4 v = *reinterpret_cast<const uint4*>(w + static_cast<size_t>(nb + wn) * Kc + wcol + wu);
                const uint32_t e[4] = {v.x ^ flip, v.y ^ flip, v.z ^ flip, v.w ^ flip};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    wT[(wu + 2 * i) * kDxP + wn] = static_cast<uint16_t>(e[i] & 0xFFFFu);
                    wT[(wu + 2 * i + 1) * kDxP + wn] = static_cast<uint16_t>(e[i] >> 16);
                }
            }
            bf16x8 af[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) af[a] = *reinterpret_cast<const bf16x8*>(dyr[a] + nb);
            __syncthreads();
            bf16x8 bfr[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) bfr[b] = *reinterpret_cast<const bf16x8*>(wT + (16 * b + fr) * kDxP + fk);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
            __syncthreads();
        }
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int col = col0 + 16 * b + fr;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = m0 + wave * 32 + 16 * a + (lane >> 4) * 4 + q;
                if (m < M) dx[static_cast<size_t>(m) * K + col] = to_bf16_bits(acc[a][b][q]);
            }
        }
}

template <int C_T>
ss1_status launch_dw_cfg(const void* x, const void* dy, const int32_t* hash, const int8_t* sign, void* dW,
                         int64_t M, const Dims& d, void* stream) {
    const dim3 grid(static_cast<unsigned>(d.G * (d.BN / kDwN)), static_cast<unsigned>((d.Kc + kDwK - 1) / kDwK));
    const size_t lds = static_cast<size_t>(d.J + d.Jc) * 4;
    hipLaunchKernelGGL((dw_kernel<C_T>), grid, dim3(256), lds, static_cast<hipStream_t>(stream),
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(dy), hash, sign,
                       static_cast<uint16_t*>(dW), (int)M, (int)d.K, (int)d.N, (int)d.J, (int)d.Jc, d.c, d.BK,
                       d.BN);
    return hipGetLastError() == hipSuccess ? SS1_OK : SS1_ERR_HIP;
}

}  // namespace

ss1_status launch_backward(const void* x, const void* W_c, const int32_t* hash, const int8_t* sign, const void* dy,
                           void* dx, void* dW, int64_t M, const Dims& d, void* stream) {
    if (dW) {
        ss1_status st;
        switch (d.c) {
            case 1: st = launch_dw_cfg<1>(x, dy, hash, sign, dW, M, d, stream); break;
            case 2: st = launch_dw_cfg<2>(x, dy, hash, sign, dW, M, d, stream); break;
            case 4: st = launch_dw_cfg<4>(x, dy, hash, sign, dW, M, d, stream); break;
            default: st = launch_dw_cfg<0>(x, dy, hash, sign, dW, M, d, stream); break;
        }
        if (st != SS1_OK) return st;
    }
    if (dx && M > 0) {
        const dim3 grid(static_cast<unsigned>((M + kDxM - 1) / kDxM), static_cast<unsigned>(d.K / kDxU));
        hipLaunchKernelGGL(dx_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                           static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(W_c), hash, sign,
                           static_cast<uint16_t*>(dx), (int)M, (int)d.K, (int)d.N, (int)d.J, (int)d.Jc, d.BK,
                           d.BN);
        if (hipGetLastError() != hipSuccess) return SS1_ERR_HIP;
    }
    return SS1_OK;
}

}  // namespace ss1
