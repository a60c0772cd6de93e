// Projection of a dense weight W [N][K] onto the SS1 sharing pattern:
// Wc[n, t*BK + u] = (1/c) * sum over the c sources j of compressed chunk t of
// sign[g][j] * W[n, j*BK + u], with g = n / BN.  This is the least-squares
// fit of W by an SS1 layer (each compressed entry is the mean of the signed
// dense entries it stands for), the reading taken for the SS1 author
// abstract's statement that pre-trained layers can be projected onto SS1.
//
// The kernel is a gather-average bound by HBM: W is read once and Wc written
// once.  A block takes a slice of one group's rows, inverts the group's hash
// in LDS, and then each thread handles 16-byte output vectors: it requests
// the c source vectors of several outputs before summing any of them
// (float32, ascending source order, as the forward's sketch), divides by c
// (IEEE division, nearest) and rounds to the output type (bf16: nearest even).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>

#include "ss1_device.h"
#include "ss1_internal.h"

namespace ss1 {

namespace {

using namespace dev;

template <typename T, int C_T, bool FROM_HASH>
__global__ __launch_bounds__(256) void project_kernel(const T* __restrict__ W, const int32_t* __restrict__ pi,
                                                      const int8_t* __restrict__ ps, T* __restrict__ Wc,
                                                      int K, int J, int Jc, int c_rt, int BK, int BN,
                                                      int rows_per_block) {
    extern __shared__ uint32_t smem[];
    uint32_t* s_src = smem;
    int* s_cnt = reinterpret_cast<int*>(smem + J);
    const int c = (C_T > 0) ? C_T : c_rt;
    const int g = blockIdx.y;
    stage_plan<FROM_HASH>(pi, ps, g, J, Jc, c, BK, s_src, s_cnt);

    constexpr bool BF16 = sizeof(T) == 2;
    constexpr int V = 16 / sizeof(T);   // elements per 16-byte vector
    constexpr int U = 4;                // outputs per thread in flight
    constexpr int CR = (C_T > 0) ? C_T : 1;
    const int Kc = Jc * BK;
    const int vpr = Kc / V;             // output vectors per row
    const int r0 = blockIdx.x * rows_per_block;
    const int nrows = min(rows_per_block, BN - r0);
    const int items = nrows * vpr;
    const size_t n0 = static_cast<size_t>(g) * BN + r0;
    const float cf = static_cast<float>(c);

    for (int base = threadIdx.x; base < items; base += U * 256) {
        size_t src_row[U], dst[U];
        int t[U], u[U];
        bool ok[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int it = base + i * 256;
            ok[i] = it < items;
            const int row = ok[i] ? it / vpr : 0;
            const int kv = (ok[i] ? it - row * vpr : 0) * V;
            t[i] = kv / BK;
            u[i] = kv - t[i] * BK;
            src_row[i] = (n0 + row) * static_cast<size_t>(K);
            dst[i] = (n0 + row) * static_cast<size_t>(Kc) + kv;
        }
        float acc[U][8];
        if constexpr (C_T > 0) {
            uint4 raw[U][CR];
            float sg[U][CR];
#pragma unroll
            for (int i = 0; i < U; ++i)
#pragma unroll
                for (int r = 0; r < C_T; ++r) {
                    const uint32_t e = s_src[t[i] * C_T + r];
                    sg[i][r] = entry_sign(e);
                    raw[i][r] = ok[i] ? *reinterpret_cast<const uint4*>(W + src_row[i] + (e & kOffMask) + u[i])
                                      : make_uint4(0, 0, 0, 0);
                }
#pragma unroll
            for (int i = 0; i < U; ++i)
#pragma unroll
                for (int r = 0; r < C_T; ++r) {
                    if constexpr (BF16) {
                        acc_bf16x8(acc[i], raw[i][r], sg[i][r], r == 0);
                    } else {
                        const float f[4] = {__uint_as_float(raw[i][r].x), __uint_as_float(raw[i][r].y),
                                            __uint_as_float(raw[i][r].z), __uint_as_float(raw[i][r].w)};
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc[i][q] = (r == 0) ? sg[i][r] * f[q] : fmaf(sg[i][r], f[q], acc[i][q]);
                    }
                }
        } else {
#pragma unroll
            for (int i = 0; i < U; ++i) {
                for (int r = 0; r < c; ++r) {
                    const uint32_t e = s_src[t[i] * c + r];
                    const float s = entry_sign(e);
                    const uint4 raw = ok[i] ? *reinterpret_cast<const uint4*>(W + src_row[i] + (e & kOffMask) + u[i])
                                            : make_uint4(0, 0, 0, 0);
                    if constexpr (BF16) {
                        acc_bf16x8(acc[i], raw, s, r == 0);
                    } else {
                        const float f[4] = {__uint_as_float(raw.x), __uint_as_float(raw.y),
                                            __uint_as_float(raw.z), __uint_as_float(raw.w)};
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[i][q] = (r == 0) ? s * f[q] : fmaf(s, f[q], acc[i][q]);
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            if (!ok[i]) continue;
#pragma unroll
            for (int q = 0; q < V; ++q) acc[i][q] = __fdiv_rn(acc[i][q], cf);
            if constexpr (BF16) {
                *reinterpret_cast<uint4*>(Wc + dst[i]) = pack_bf16x8(acc[i]);
            } else {
                *reinterpret_cast<float4*>(Wc + dst[i]) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
            }
        }
    }
}

template <typename T, int C_T>
ss1_status launch_project_cfg(const void* W, const int32_t* hash, const int8_t* sign, const Dims& d, void* Wc,
                              void* stream) {
    constexpr int V = 16 / sizeof(T);
    const long long vpr = d.Kc / V;
    // about 4096 output vectors per block, whole rows, inside one group
    const int rows = static_cast<int>(std::max<long long>(1, std::min<long long>(d.BN, 4096 / vpr)));
    const unsigned bx = static_cast<unsigned>((d.BN + rows - 1) / rows);
    const size_t lds = static_cast<size_t>(d.J + d.Jc) * 4;
    hipLaunchKernelGGL((project_kernel<T, C_T, true>), dim3(bx, static_cast<unsigned>(d.G)), dim3(256), lds,
                       static_cast<hipStream_t>(stream), static_cast<const T*>(W), hash, sign, static_cast<T*>(Wc),
                       (int)d.K, (int)d.J, (int)d.Jc, d.c, d.BK, d.BN, rows);
    return hipGetLastError() == hipSuccess ? SS1_OK : SS1_ERR_HIP;
}

template <typename T>
ss1_status launch_project_t(const void* W, const int32_t* hash, const int8_t* sign, const Dims& d, void* Wc,
                            void* stream) {
    switch (d.c) {
        case 1: return launch_project_cfg<T, 1>(W, hash, sign, d, Wc, stream);
        case 2: return launch_project_cfg<T, 2>(W, hash, sign, d, Wc, stream);
        case 4: return launch_project_cfg<T, 4>(W, hash, sign, d, Wc, stream);
        case 8: return launch_project_cfg<T, 8>(W, hash, sign, d, Wc, stream);
        default: return launch_project_cfg<T, 0>(W, hash, sign, d, Wc, stream);
    }
}

}  // namespace

ss1_status launch_project(const void* W, int32_t dtype, const int32_t* hash, const int8_t* sign, const Dims& d,
                          void* Wc, void* stream) {
    return dtype == SS1_BF16 ? launch_project_t<uint16_t>(W, hash, sign, d, Wc, stream)
                             : launch_project_t<float>(W, hash, sign, d, Wc, stream);
}

}  // namespace ss1
