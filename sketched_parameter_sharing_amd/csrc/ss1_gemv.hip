// Decode-shape SS1 forward as a matrix-vector product (M <= 4 tokens).
//
// The SS1 layer forward of "Sketch Structured Transforms" (the layer
// definition: each group's input sketch times the group's rows of W_c) does,
// for a handful of tokens, two floating-point operations per weight and token:
// no matrix-core shape, and the time is the HBM stream of W_c.  The kernel is
// built so that each block has its whole share of W_c in flight at once:
//   * a block takes R consecutive rows of one group; thread t of its NT
//     threads (NT a multiple of 64, sized to the row) owns the 8-element
//     slices t, t + NT, t + 2 NT, ... of the compressed row (Q of them), so
//     each row is read as whole contiguous 16-byte pieces;
//   * the thread reads its entries of the group's plan into registers, then
//     issues the loads of its R x Q weight slices, and only then waits for the
//     plan (loads complete in order, so the plan's wait leaves the weights in
//     flight), stages the plan in LDS and gathers its sketch slices for each
//     token from the c source chunks of x (float32 signed sums rounded to
//     bf16, the rounding of the other sketch kernels);
//   * each thread multiplies in float32; the R x MT partial sums are reduced
//     across the wave by lane exchanges that halve the values carried at each
//     step, then across the block's waves through LDS, all in a fixed order.
#include <algorithm>

#include "ss1_device.h"

namespace ss1 {
namespace {

using namespace dev;

constexpr int kGemvMaxThreads = 1024;

// Eight consecutive weights of one row: 16 bytes of bf16 or 8 of E4M3.
template <bool W8>
struct WSlice {
    uint4 v;
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t s) {
        v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, 16 * s, 0, kNonTemporal));
    }
    __device__ __forceinline__ uint4 bf16() const { return v; }
};
template <>
struct WSlice<true> {
    uint2 v;
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t s) {
        v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, 8 * s, 0, kNonTemporal));
    }
    __device__ __forceinline__ uint4 bf16() const { return fp8x8_to_bf16x8(v); }
};

// Lane exchange partner^off inside a row of 16 lanes with DPP moves (no LDS
// round trip): xor 1 and 2 are quad permutes; xor 4 and 8 take the value
// from lane i + off where lane bit off is clear (row_shl) and from i - off
// where it is set (row_shr).
template <int OFF>
__device__ __forceinline__ float dpp_xor(float v, bool up) {
    const int b = __builtin_bit_cast(int, v);
    if constexpr (OFF == 1) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, b, 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
    } else if constexpr (OFF == 2) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, b, 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
    } else {
        const int from_above = __builtin_amdgcn_update_dpp(0, b, 0x100 + OFF, 0xF, 0xF, true);  // row_shl
        const int from_below = __builtin_amdgcn_update_dpp(0, b, 0x110 + OFF, 0xF, 0xF, true);  // row_shr
        return __builtin_bit_cast(float, up ? from_below : from_above);
    }
}

// The value of lane (this lane) ^ OFF: DPP inside a row of 16 lanes, a
// permute through the LDS crossbar across rows.
template <int OFF>
__device__ __forceinline__ float lane_xor(float v, bool up) {
    if constexpr (OFF <= 8) {
        return dpp_xor<OFF>(v, up);
    } else {
        return __shfl_xor(v, OFF);
    }
}

// One halving step at lane bit OFF: the lane keeps half of its 2 H values
// (the upper half when its bit OFF is set) and adds the partner's copy of
// that half; with H == 0 a plain butterfly on one value.
template <int OFF, int H, int V>
__device__ __forceinline__ void halve(float (&v)[V], int lane, int& idx) {
    const bool up = (lane & OFF) != 0;
    if constexpr (H == 0) {
        v[0] += lane_xor<OFF>(v[0], up);
    } else {
#pragma unroll
        for (int i = 0; i < H; ++i) {
            const float keep = up ? v[i + H] : v[i];
            const float give = up ? v[i] : v[i + H];
            v[i] = keep + lane_xor<OFF>(give, up);
        }
        idx = 2 * idx + (up ? 1 : 0);
    }
}

// R rows, MT token slots (tokens >= M are zero), Q slices per thread, C_T
// sources per compressed chunk (0: c at run time); blockDim.x threads.
template <int R, int MT, int Q, int C_T, bool W8, bool FROM_HASH>
__global__ __launch_bounds__(kGemvMaxThreads) void gemv_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                  const int32_t* __restrict__ pi, const int8_t* __restrict__ ps,
                                                  uint16_t* __restrict__ y, int M, int K, int N, int J, int Jc,
                                                  int c_rt, int BK, int BN, int act,
                                                  const float* __restrict__ wscale) {
    const int NT = blockDim.x;
    const int NW = NT / 64;
    constexpr int V = R * MT;  // partial sums per thread, value i = r * MT + m
    static_assert((V & (V - 1)) == 0 && V <= 32, "V is a power of two, at most 32");
    constexpr int PJ = kPlanPerThread;
    extern __shared__ uint32_t smem[];
    float* red = reinterpret_cast<float*>(smem);  // [NW][V]
    uint32_t* s_src = smem + NW * V;
    int* s_cnt = reinterpret_cast<int*>(s_src + J);

    const int c = (C_T > 0) ? C_T : c_rt;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n0 = blockIdx.x * R;
    const int g = n0 / BN;
    const int Kc = Jc * BK;
    const int S8 = Kc >> 3;

    // 1. this thread's plan entries
    int32_t iv[PJ];
    int8_t sv[PJ];
    fetch_plan_regs<PJ>(pi, ps, g, J, iv, sv);

    // 2. all of this thread's weight slices (slices past the row read zeros)
    constexpr int WB = W8 ? 1 : 2;
    WSlice<W8> wr[R][Q];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const __amdgpu_buffer_rsrc_t wrs =
            make_rsrc(reinterpret_cast<const uint8_t*>(w) + static_cast<size_t>(n0 + r) * Kc * WB,
                      static_cast<uint32_t>(Kc) * WB);
#pragma unroll
        for (int q = 0; q < Q; ++q) wr[r][q].load(wrs, static_cast<uint32_t>(tid + q * NT));
    }

    // 3. plan in LDS
    stage_plan_regs<FROM_HASH, PJ>(iv, sv, J, Jc, c, BK, s_src, s_cnt);

    // 4. per slice: the sketch of each token, then its products with the R
    // rows' weights
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, static_cast<uint32_t>(M) * K * 2);
    float v[V];
#pragma unroll
    for (int i = 0; i < V; ++i) v[i] = 0.0f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int s = tid + q * NT;
        const bool ok = s < S8;
        const int k = 8 * (ok ? s : 0);
        const int t = k / BK;
        const int u0 = k - t * BK;
        // token rows past M and slices past the row read zeros; every token's
        // gathers are issued before the first is used
        float z[MT][8];
        if constexpr (C_T > 0) {
            uint32_t e[C_T];
#pragma unroll
            for (int r = 0; r < C_T; ++r) e[r] = s_src[t * C_T + r];
            uint4 raw[MT][C_T];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const uint32_t base = ok ? static_cast<uint32_t>(m * K + u0) * 2 : kOutOfRange;
#pragma unroll
                for (int r = 0; r < C_T; ++r) raw[m][r] = buf_load16(xrs, base + (e[r] & kOffMask) * 2, 0);
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                float a[8];
#pragma unroll
                for (int r = 0; r < C_T; ++r) acc_bf16x8(a, raw[m][r], entry_sign(e[r]), r == 0);
#pragma unroll
                for (int i = 0; i < 8; ++i) z[m][i] = round_to_bf16(a[i]);
            }
        } else {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const uint32_t base = ok ? static_cast<uint32_t>(m * K + u0) * 2 : kOutOfRange;
                float a[8];
                for (int r = 0; r < c; ++r) {
                    const uint32_t e = s_src[t * c + r];
                    acc_bf16x8(a, buf_load16(xrs, base + (e & kOffMask) * 2, 0), entry_sign(e), r == 0);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) z[m][i] = round_to_bf16(a[i]);
            }
        }
        for (int r = 0; r < R; ++r) {
            const uint4 wb = wr[r][q].bf16();
            const uint32_t ww[4] = {wb.x, wb.y, wb.z, wb.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float lo = bf16_lo(ww[i]);
                const float hi = bf16_hi(ww[i]);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    v[r * MT + m] = fmaf(lo, z[m][2 * i], v[r * MT + m]);
                    v[r * MT + m] = fmaf(hi, z[m][2 * i + 1], v[r * MT + m]);
                }
            }
        }
    }

    // 5. reduction over the wave.  While a lane carries several values, each
    // exchange (lane bits 1, 2, 4, 8, 16 in turn) hands half of them to the
    // partner lane and keeps the other half; the lane's remaining value index
    // collects those lane bits, lowest first as the most significant.  Then
    // plain butterflies over the remaining lane bits; lanes 0 .. V-1 hold the
    // wave's V sums.
    int idx = 0;
    halve<1, V / 2>(v, lane, idx);
    halve<2, V / 4>(v, lane, idx);
    halve<4, V / 8>(v, lane, idx);
    halve<8, V / 16>(v, lane, idx);
    halve<16, V / 32>(v, lane, idx);
    halve<32, 0>(v, lane, idx);
    if (lane < V) red[wave * V + idx] = v[0];
    __syncthreads();

    // 6. sum over the waves, epilogue
    if (tid < V) {
        float sum = red[tid];
#pragma unroll
        for (int u = 1; u < NW; ++u) sum += red[u * V + tid];
        const int r = tid / MT;
        const int m = tid - r * MT;
        if (m < M) {
            const int n = n0 + r;
            const float ws = W8 ? wscale[n] : 1.0f;
            y[static_cast<size_t>(m) * N + n] = to_bf16_bits(apply_act(sum * ws, act));
        }
    }
}

inline ss1_status launch_status() {
    return hipGetLastError() == hipSuccess ? SS1_OK : SS1_ERR_HIP;
}

struct GemvCfg {
    int MT, Q, R, NT;  // MT == 0: not supported
};

// Token slots (1, 2 or 4); threads and slices per thread: one 8-element slice
// per thread up to 1024 threads (NT the row's slice count rounded up to a
// whole wave), else 1024 threads with 2, 4 or 8 slices (MT * Q <= 8, so the
// sketch stays in 64 registers); rows per block: 8 weight loads of 16 bytes
// per thread (16 of 8 bytes for fp8), with at most 32 partial sums (rows x
// token slots) per thread.
inline GemvCfg gemv_config(const ForwardArgs& a) {
    const Dims& d = a.d;
    GemvCfg cfg{0, 0, 0, 0};
    if (a.M > 4 || d.K > (int64_t{1} << 26)) return cfg;  // 32-bit byte offsets into x
    const int64_t s8 = d.Kc / 8;
    if (s8 < 64) return cfg;  // rows shorter than one wave's slices
    const int MT = a.M <= 1 ? 1 : (a.M <= 2 ? 2 : 4);
    int Q = 1;
    while (static_cast<int64_t>(Q) * kGemvMaxThreads < s8) Q *= 2;
    if (MT * Q > 8) return cfg;
    const int64_t per_thread = (s8 + Q - 1) / Q;
    const int NT = static_cast<int>((per_thread + 63) / 64 * 64);
    if (d.J > static_cast<int64_t>(NT) * kPlanPerThread) return cfg;
    // four token slots take about 80 registers, so a block of more than 512
    // threads runs alone on its compute unit (Llama down, M = 3 or 4: 20.5 us
    // against 17.1 us on the small-M kernel)
    if (MT == 4 && NT > 512) return cfg;
    int R = std::min((a.w_fp8 ? 16 : 8) / Q, 32 / MT);
    if (R < 1) R = 1;
    if (d.BN % R) return cfg;
    cfg.MT = MT;
    cfg.Q = Q;
    cfg.R = R;
    cfg.NT = NT;
    return cfg;
}

template <int R, int MT, int Q, int C_T, bool W8, bool FROM_HASH>
ss1_status launch_gemv_cfg(const ForwardArgs& a, const GemvCfg& cfg) {
    const Dims& d = a.d;
    const long long blocks = d.N / R;
    if (blocks > 0x7FFFFFFFLL) return SS1_ERR_SHAPE;
    const size_t lds = static_cast<size_t>(cfg.NT / 64) * R * MT * 4 + static_cast<size_t>(d.J + d.Jc) * 4;
    hipLaunchKernelGGL((gemv_kernel<R, MT, Q, C_T, W8, FROM_HASH>), dim3(static_cast<unsigned>(blocks)),
                       dim3(cfg.NT), lds, static_cast<hipStream_t>(a.stream), static_cast<const uint16_t*>(a.x),
                       static_cast<const uint16_t*>(a.w), a.plan_i, a.plan_s, static_cast<uint16_t*>(a.y), (int)a.M,
                       (int)d.K, (int)d.N, (int)d.J, (int)d.Jc, d.c, d.BK, d.BN, a.act, a.wscale);
    return launch_status();
}

// R as gemv_config sets it; a table of the (MT, Q) pairs it allows.
template <int MT, int Q, int C_T, bool W8, bool FROM_HASH>
ss1_status launch_gemv_r(const ForwardArgs& a, const GemvCfg& cfg) {
    constexpr int R0 = std::min((W8 ? 16 : 8) / Q, 32 / MT);
    constexpr int R = R0 < 1 ? 1 : R0;
    if (cfg.R != R) return SS1_ERR_ALGO;
    return launch_gemv_cfg<R, MT, Q, C_T, W8, FROM_HASH>(a, cfg);
}

template <int C_T, bool W8, bool FROM_HASH>
ss1_status launch_gemv_c(const ForwardArgs& a, const GemvCfg& cfg) {
    switch (cfg.MT * 16 + cfg.Q) {
        case 16 + 1: return launch_gemv_r<1, 1, C_T, W8, FROM_HASH>(a, cfg);
        case 16 + 2: return launch_gemv_r<1, 2, C_T, W8, FROM_HASH>(a, cfg);
        case 16 + 4: return launch_gemv_r<1, 4, C_T, W8, FROM_HASH>(a, cfg);
        case 16 + 8: return launch_gemv_r<1, 8, C_T, W8, FROM_HASH>(a, cfg);
        case 32 + 1: return launch_gemv_r<2, 1, C_T, W8, FROM_HASH>(a, cfg);
        case 32 + 2: return launch_gemv_r<2, 2, C_T, W8, FROM_HASH>(a, cfg);
        case 32 + 4: return launch_gemv_r<2, 4, C_T, W8, FROM_HASH>(a, cfg);
        case 64 + 1: return launch_gemv_r<4, 1, C_T, W8, FROM_HASH>(a, cfg);
        case 64 + 2: return launch_gemv_r<4, 2, C_T, W8, FROM_HASH>(a, cfg);
        default: return SS1_ERR_ALGO;
    }
}

template <bool W8, bool FROM_HASH>
ss1_status launch_gemv_t(const ForwardArgs& a) {
    const GemvCfg cfg = gemv_config(a);
    if (cfg.MT == 0) return SS1_ERR_ALGO;
    switch (a.d.c) {
        case 1: return launch_gemv_c<1, W8, FROM_HASH>(a, cfg);
        case 2: return launch_gemv_c<2, W8, FROM_HASH>(a, cfg);
        case 4: return launch_gemv_c<4, W8, FROM_HASH>(a, cfg);
        case 8: return launch_gemv_c<8, W8, FROM_HASH>(a, cfg);
        default: return launch_gemv_c<0, W8, FROM_HASH>(a, cfg);
    }
}

}  // namespace

bool gemv_supported(const ForwardArgs& a) {
    return a.dtype == SS1_BF16 && a.d.BN % 16 == 0 && (!a.w_fp8 || a.form == PlanForm::Hash) &&
           gemv_config(a).MT > 0;
}

ss1_status launch_gemv(const ForwardArgs& a) {
    if (a.w_fp8) return a.form == PlanForm::Hash ? launch_gemv_t<true, true>(a) : SS1_ERR_ALGO;
    return a.form == PlanForm::Hash ? launch_gemv_t<false, true>(a) : launch_gemv_t<false, false>(a);
}

}  // namespace ss1
