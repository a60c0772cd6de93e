// Decode forward for up to 16 tokens whose input rows fit in LDS (16*K bf16):
// y = z_g W_c,g^T per group, the sketch z_g of the SS1 summary page,
// "Approach" (signed sums of the input chunks that hash to each compressed
// chunk), rounded to bf16 and multiplied on the bf16 matrix cores.
//
// At 16 tokens the layer moves its compressed weight once (58.7 MB for the
// Llama-3-8B gate/up projection) and little else, so the kernel is built to
// keep that stream going: a block is one neuron group (BN = 16*RB neurons)
// and all its compressed columns, 16 waves each taking a sixteenth of the
// columns.  Each wave issues all of its weight loads (RB x 4 loads of 16 bytes
// per lane, 32-wide k-steps, whole 128-byte lines) before it waits for
// anything; the input rows
// reach LDS once per block by direct buffer-to-LDS loads (rows past M read
// zeros) and the sketch of every k-step is formed from LDS, so no input
// element is gathered from L2 per k-step.  The plan entries are read into
// registers first, since loads return in the order issued.
//
// Per k-step a lane forms 8 sketch elements (token lane%16, columns
// 8*(lane/16) ..) in float32 from the c source chunks, rounds them to bf16,
// and feeds RB MFMAs 16x16x32 with the weight operand of each 16-neuron row
// block.  The weights of two consecutive k-steps (64 columns, one 128-byte
// line per row) of a row block come in two loads of 8 rows each, and two
// lane rotations inside each 16-lane row turn them into the two steps'
// operands.  The partial tiles of the 16
// waves are summed in LDS in wave order, and each lane stores 4 consecutive
// neurons of one token (8 bytes).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>

#include "ss1_device.h"
#include "ss1_dma.h"
#include "ss1_internal.h"

namespace ss1 {

namespace {

using namespace dev;

// 16 waves of 4 k-steps measured 2.7% ahead of 8 waves of 8 on the Llama-3-8B
// gate/up decode shape (19.6 against 20.1 us); the bytes in flight per block
// are the same
constexpr int kDecWaves = 16;
constexpr int kDecSteps = 4;  // k-steps per wave whose weight loads are in flight together
static_assert(kDecSteps % 2 == 0, "k-steps come in pairs of one 128-byte line");

// LDS of a decode launch: the x tile (or the wave partials, which reuse it)
// and the group's plan (J entries plus Jc counters).
size_t decode_lds(int64_t K, const Dims& d) {
    const size_t xb = static_cast<size_t>(16) * K * 2;
    const size_t red = static_cast<size_t>(d.BN / 16) * kDecWaves * 64 * 16;
    return std::max(xb, red) + static_cast<size_t>(d.J + d.Jc) * 4;
}

template <int RB, int C_T, bool FROM_HASH>
__global__ __launch_bounds__(kDecWaves * 64) void decode_kernel(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ w,
                                                                const int32_t* __restrict__ pi,
                                                                const int8_t* __restrict__ ps,
                                                                uint16_t* __restrict__ y, int M, int K, int N,
                                                                int J, int Jc, int c_rt, int BK, int act) {
    constexpr int NW = kDecWaves;
    constexpr int BN = 16 * RB;
    extern __shared__ __attribute__((aligned(16))) uint8_t dec_smem[];
    const int xbytes = 16 * K * 2;
    const int redbytes = RB * NW * 64 * 16;
    uint16_t* sx = reinterpret_cast<uint16_t*>(dec_smem);
    f32x4* red = reinterpret_cast<f32x4*>(dec_smem);  // [RB][NW][64], over the x tile once it is read
    uint32_t* s_src = reinterpret_cast<uint32_t*>(dec_smem + (xbytes > redbytes ? xbytes : redbytes));
    int* s_cnt = reinterpret_cast<int*>(s_src + J);

    const int c = (C_T > 0) ? C_T : c_rt;
    const int g = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int Kc = Jc * BK;

    // (1) this thread's plan entries, first: loads return in the order issued
    int32_t iv[kPlanPerThread];
    int8_t sv[kPlanPerThread];
    fetch_plan_regs<kPlanPerThread>(pi, ps, g, J, iv, sv);

    // (2) the input rows into LDS.  Row t holds K bf16 as K/8 pieces of 16
    // bytes; piece p sits at slot p ^ t (t < 16), so the 16 lanes that read
    // one column of rows 0..15 hit 16 distinct bank groups.  K % 512 == 0:
    // a row is a whole number of wave-wide loads (64 pieces each), and the 16
    // rows' loads split evenly over the 16 waves.
    const int lpr = K / 512;  // wave-wide loads per row
    const i32x4 xrs = dma_rsrc(x, static_cast<uint32_t>(M * K * 2));
    const uint32_t xlds = lds_address(dec_smem);
    for (int i = wave; i < 16 * lpr; i += NW) {
        const int t = i / lpr;
        const int pb = (i - t * lpr) * 64;
        const uint32_t voff = static_cast<uint32_t>(t * K * 2 + ((pb + lane) ^ t) * 16);
        lds_dma16(xrs, xlds + static_cast<uint32_t>(i * 1024), voff, 0u);
    }

    // (3) this wave's weight loads: k-steps [sb, se) of the group's Kc/32,
    // in pairs (sb even).  Each load covers 8 rows x 128 bytes, whole lines
    // (on the Llama-3-8B gate/up decode shape the whole layer took 19.3 us
    // with loads of 16 rows x 64 bytes in the operand layout itself, 15.9
    // with these and no rotations); lane l reads row l%8 (plus 8 for the
    // pair's second load) at piece (l/16) + 4*((l/8)%2).  A pair that starts
    // before se is loaded whole (a second step at or past se is never
    // multiplied); columns past Kc fall in the next row, or past the extent
    // on the last row, which reads zeros.
    const int S = Kc / 32;
    const int SP = (S + 1) / 2;
    const int sb = 2 * ((SP * wave) / NW);
    const int se = min(S, 2 * ((SP * (wave + 1)) / NW));
    const __amdgpu_buffer_rsrc_t wrs =
        make_rsrc(w + static_cast<size_t>(g) * BN * Kc, static_cast<uint32_t>(BN * Kc * 2));
    const uint32_t wl = pair_load_offset(lane, Kc);
    uint4 wv[kDecSteps][RB];  // [2v][rb]: rows 0..7 of pair v, [2v+1][rb]: rows 8..15
    auto load_w = [&](int s0) {
#pragma unroll
        for (int u = 0; u < kDecSteps; ++u)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int p0 = s0 + (u & ~1);  // first step of the pair
                const uint32_t off =
                    (p0 < se) ? wl + static_cast<uint32_t>(((rb * 16 + 8 * (u & 1)) * Kc + p0 * 32) * 2) : kOutOfRange;
                wv[u][rb] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, kNonTemporal));
            }
    };
    load_w(sb);

    // (4) the plan into LDS from the registers of (1); then every wave's part
    // of the x tile must have landed (the weight loads may stay in flight).
    // The count in the wait assumes the RB * kDecSteps weight loads above are
    // issued before it: the compiler may move buffer loads below an inline-asm
    // wait (it did so for loads placed right before one), but not below the
    // LDS barriers of stage_plan_regs, which sit between them here; the
    // parity tests read all 16 rows at M = 16, where a short wait would show.
    stage_plan_regs<FROM_HASH, kPlanPerThread>(iv, sv, J, Jc, c, BK, s_src, s_cnt);
    dma_stage_barrier<RB * kDecSteps>();

    // (5) sketch and MFMA per k-step
    const int tok = lane & 15;
    const int kq = (lane >> 4) * 8;
    const uint32_t lo8 = pair_lane_mask(lane);
    const uint16_t* xrow = sx + tok * K;
    f32x4 acc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = sb; s0 < se; s0 += kDecSteps) {
        if (s0 != sb) load_w(s0);
        // the sketches of all the batch's steps first (LDS and vector work
        // only), then the MFMAs in the order the weights arrive
        uint4 z[kDecSteps];
#pragma unroll
        for (int u = 0; u < kDecSteps; ++u) {
            const int kc = min(s0 + u, se - 1) * 32 + kq;  // compressed column of this lane's 8 elements
            const int t = kc / BK;
            const int u0 = kc - t * BK;
            float a[8];
            for (int r = 0; r < c; ++r) {
                const uint32_t e = s_src[t * c + r];
                const int piece = static_cast<int>(((e & kOffMask) + static_cast<uint32_t>(u0)) >> 3);
                const uint4 raw = *reinterpret_cast<const uint4*>(xrow + ((piece ^ tok) << 3));
                acc_bf16x8(a, raw, entry_sign(e), r == 0);
            }
            z[u] = pack_bf16x8(a);
        }
#pragma unroll
        for (int u = 0; u < kDecSteps; u += 2) {
            if (s0 + u < se) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    uint4 t0, t1;
                    pair_operands(wv[u][rb], wv[u + 1][rb], lo8, t0, t1);
                    acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t0),
                                                                       __builtin_bit_cast(bf16x8, z[u]), acc[rb],
                                                                       0, 0, 0);
                    if (s0 + u + 1 < se)
                        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t1),
                                                                           __builtin_bit_cast(bf16x8, z[u + 1]),
                                                                           acc[rb], 0, 0, 0);
                }
            }
        }
    }

    // (6) partial tiles summed over the waves in wave order; lane l of wave
    // rb < RB holds neurons rb*16 + 4*(l/16) .. +3 of token l%16
    lds_barrier();  // every wave is done with the x tile
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) red[(rb * NW + wave) * 64 + lane] = acc[rb];
    lds_barrier();
    if (wave < RB) {
        const f32x4* rp = red + wave * NW * 64;
        f32x4 sum = rp[lane];
        for (int v = 1; v < NW; ++v) {
            const f32x4 p = rp[v * 64 + lane];
            sum[0] += p[0];
            sum[1] += p[1];
            sum[2] += p[2];
            sum[3] += p[3];
        }
        if (tok < M) {
            const int n = g * BN + wave * 16 + 4 * (lane >> 4);
            uint2 o;
            o.x = pack_bf16(apply_act(sum[0], act), apply_act(sum[1], act));
            o.y = pack_bf16(apply_act(sum[2], act), apply_act(sum[3], act));
            *reinterpret_cast<uint2*>(y + static_cast<size_t>(tok) * N + n) = o;
        }
    }
}

// ------------------------------------------------------- column-split decode
// For decode layers whose 16 input rows do not fit in LDS (or whose groups are
// too few to fill the compute units): block (g, q) takes neuron group g and
// the q-th of Q equal slices of its compressed columns.  Each block stages in
// LDS only the input chunks that its slice's compressed chunks sum (16 rows x
// K/Q bf16), issues its weight loads first (whole lines, as the decode
// kernel), and writes its float32 partial tile to part[q][m][n]; the slices
// are then summed in order q = 0 .. Q-1 by split_sum_kernel.
//
// Order of a block's work: plan entries into registers, every weight load of
// the wave, the plan into LDS, the input chunks into LDS (their offsets come
// from the plan), one wait for all of them, then the sketches and MFMAs.
// Loads complete in issue order, so the input chunks are waited for after
// the weights; the weights, not the input chunks, set the time.
template <int RB, int C_T, bool FROM_HASH>
__global__ __launch_bounds__(kDecWaves * 64) void split_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ w,
                                                               const int32_t* __restrict__ pi,
                                                               const int8_t* __restrict__ ps,
                                                               float* __restrict__ part, int M, int K, int N,
                                                               int J, int Jc, int c_rt, int BK, int Q) {
    constexpr int NW = kDecWaves;
    constexpr int BN = 16 * RB;
    extern __shared__ __attribute__((aligned(16))) uint8_t spl_smem[];
    const int c = (C_T > 0) ? C_T : c_rt;
    const int g = blockIdx.x / Q;
    const int q = blockIdx.x - g * Q;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int Kc = Jc * BK;
    const int Ks = Kc / Q;            // compressed columns of the slice
    const int t0 = q * (Ks / BK);     // its first compressed chunk
    const int ppc = BK / 8;           // 16-byte pieces per chunk
    const int rowp = (Ks / BK) * c * ppc;  // pieces per staged input row (K/Q/8)
    const int xbytes = 16 * rowp * 16;
    const int redbytes = RB * NW * 64 * 16;
    f32x4* red = reinterpret_cast<f32x4*>(spl_smem);  // [RB][NW][64], over the input tile once it is read
    uint32_t* s_src = reinterpret_cast<uint32_t*>(spl_smem + (xbytes > redbytes ? xbytes : redbytes));
    int* s_cnt = reinterpret_cast<int*>(s_src + J);

    // (1) plan entries into registers
    int32_t iv[kPlanPerThread];
    int8_t sv[kPlanPerThread];
    fetch_plan_regs<kPlanPerThread>(pi, ps, g, J, iv, sv);

    // (2) this wave's weight loads: k-steps [sb, se) of the slice's Ks/32 in
    // pairs, as in the decode kernel
    const int S = Ks / 32;
    const int SP = (S + 1) / 2;
    const int sb = 2 * ((SP * wave) / NW);
    const int se = min(S, 2 * ((SP * (wave + 1)) / NW));
    const __amdgpu_buffer_rsrc_t wrs =
        make_rsrc(w + static_cast<size_t>(g) * BN * Kc, static_cast<uint32_t>(BN * Kc * 2));
    const uint32_t wl = pair_load_offset(lane, Kc) + static_cast<uint32_t>(q * Ks * 2);
    uint4 wv[kDecSteps][RB];
    auto load_w = [&](int s0) {
#pragma unroll
        for (int u = 0; u < kDecSteps; ++u)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int p0 = s0 + (u & ~1);
                const uint32_t off =
                    (p0 < se) ? wl + static_cast<uint32_t>(((rb * 16 + 8 * (u & 1)) * Kc + p0 * 32) * 2) : kOutOfRange;
                wv[u][rb] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, kNonTemporal));
            }
    };
    load_w(sb);

    // (3) the plan into LDS
    stage_plan_regs<FROM_HASH, kPlanPerThread>(iv, sv, J, Jc, c, BK, s_src, s_cnt);

    // (4) the slice's input chunks into LDS: row t (token) holds, for local
    // chunk lc = (compressed chunk - t0) * c + r, source r of that compressed
    // chunk, as ppc pieces of 16 bytes; piece p of row t sits at slot p ^ t.
    // An absent source, and rows past M, read zeros.
    const int lpr = rowp / 64;  // wave-wide loads per row
    const i32x4 xrs = dma_rsrc(x, static_cast<uint32_t>(M * K * 2));
    const uint32_t xlds = lds_address(spl_smem);
    for (int i = wave; i < 16 * lpr; i += NW) {
        const int t = i / lpr;
        const int pidx = (i - t * lpr) * 64 + lane;  // LDS slot of this lane
        const int p = pidx ^ t;                      // the piece it holds
        const int lc = p / ppc;
        const int e = p - lc * ppc;
        const uint32_t ent = s_src[(t0 + lc / c) * c + lc % c];
        const uint32_t voff = (ent & kAbsent) ? kDmaAbsent
                                              : static_cast<uint32_t>((t * K + (ent & kOffMask) + e * 8) * 2);
        lds_dma16(xrs, xlds + static_cast<uint32_t>(i * 1024), voff, 0u);
    }
    dma_stage_barrier<0>();

    // (5) sketch and MFMA per k-step
    const int tok = lane & 15;
    const int kq = (lane >> 4) * 8;
    const uint32_t lo8 = pair_lane_mask(lane);
    const uint4* xrow = reinterpret_cast<const uint4*>(spl_smem) + tok * rowp;
    f32x4 acc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = sb; s0 < se; s0 += kDecSteps) {
        if (s0 != sb) load_w(s0);
        uint4 z[kDecSteps];
#pragma unroll
        for (int u = 0; u < kDecSteps; ++u) {
            const int kc = min(s0 + u, se - 1) * 32 + kq;  // column inside the slice
            const int tl = kc / BK;                         // local compressed chunk
            const int u0 = kc - tl * BK;
            float a[8];
            for (int r = 0; r < c; ++r) {
                const uint32_t ent = s_src[(t0 + tl) * c + r];
                const int piece = (tl * c + r) * ppc + (u0 >> 3);
                acc_bf16x8(a, xrow[piece ^ tok], entry_sign(ent), r == 0);
            }
            z[u] = pack_bf16x8(a);
        }
#pragma unroll
        for (int u = 0; u < kDecSteps; u += 2) {
            if (s0 + u < se) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    uint4 w0, w1;
                    pair_operands(wv[u][rb], wv[u + 1][rb], lo8, w0, w1);
                    acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w0),
                                                                       __builtin_bit_cast(bf16x8, z[u]), acc[rb],
                                                                       0, 0, 0);
                    if (s0 + u + 1 < se)
                        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w1),
                                                                           __builtin_bit_cast(bf16x8, z[u + 1]),
                                                                           acc[rb], 0, 0, 0);
                }
            }
        }
    }

    // (6) the waves' partial tiles summed in wave order; lane l of wave
    // rb < RB holds neurons rb*16 + 4*(l/16) .. +3 of token l%16
    lds_barrier();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) red[(rb * NW + wave) * 64 + lane] = acc[rb];
    lds_barrier();
    if (wave < RB) {
        const f32x4* rp = red + wave * NW * 64;
        f32x4 sum = rp[lane];
        for (int v = 1; v < NW; ++v) {
            const f32x4 pv = rp[v * 64 + lane];
            sum[0] += pv[0];
            sum[1] += pv[1];
            sum[2] += pv[2];
            sum[3] += pv[3];
        }
        if (tok < M) {
            const int n = g * BN + wave * 16 + 4 * (lane >> 4);
            *reinterpret_cast<float4*>(part + (static_cast<size_t>(q) * M + tok) * N + n) =
                make_float4(sum[0], sum[1], sum[2], sum[3]);
        }
    }
}

// y[m][n] = act(sum over q = 0 .. Q-1, in that order, of part[q][m][n]),
// rounded to bf16; one thread per 4 consecutive outputs.
__global__ __launch_bounds__(256) void split_sum_kernel(const float* __restrict__ part, uint16_t* __restrict__ y,
                                                        int M, int N, int Q, int act) {
    const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
    const long long quads = static_cast<long long>(M) * N / 4;
    if (i >= quads) return;
    const size_t plane = static_cast<size_t>(M) * N;
    const float4* p = reinterpret_cast<const float4*>(part) + i;
    float4 s = p[0];
    for (int k = 1; k < Q; ++k) {
        const float4 v = p[k * (plane / 4)];
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    uint2 o;
    o.x = pack_bf16(apply_act(s.x, act), apply_act(s.y, act));
    o.y = pack_bf16(apply_act(s.z, act), apply_act(s.w, act));
    reinterpret_cast<uint2*>(y)[i] = o;
}

template <int RB, int C_T, bool FROM_HASH>
ss1_status launch_decode_cfg(const ForwardArgs& a) {
    const Dims& d = a.d;
    const size_t lds = decode_lds(d.K, d);
    auto kern = &decode_kernel<RB, C_T, FROM_HASH>;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds)) != hipSuccess)
        return SS1_ERR_HIP;
    hipLaunchKernelGGL((decode_kernel<RB, C_T, FROM_HASH>), dim3(static_cast<unsigned>(d.G)), dim3(kDecWaves * 64),
                       lds, static_cast<hipStream_t>(a.stream), static_cast<const uint16_t*>(a.x),
                       static_cast<const uint16_t*>(a.w), a.plan_i, a.plan_s, static_cast<uint16_t*>(a.y),
                       static_cast<int>(a.M), static_cast<int>(d.K), static_cast<int>(d.N), static_cast<int>(d.J),
                       static_cast<int>(d.Jc), d.c, d.BK, a.act);
    return hipGetLastError() == hipSuccess ? SS1_OK : SS1_ERR_HIP;
}

template <int RB, bool FROM_HASH>
ss1_status launch_decode_rb(const ForwardArgs& a) {
    if (a.d.c == 2) return launch_decode_cfg<RB, 2, FROM_HASH>(a);
    return launch_decode_cfg<RB, 0, FROM_HASH>(a);
}

int max_lds() {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 64 * 1024;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0)
        return 64 * 1024;
    return v;
}

// LDS of a split launch: the staged input chunks (16 rows of K/Q bf16) or the
// wave partials, plus the group's plan (J entries and Jc counters).
size_t split_lds(int Q, const Dims& d) {
    const size_t xb = static_cast<size_t>(16) * (d.K / Q) * 2;
    const size_t red = static_cast<size_t>(d.BN / 16) * kDecWaves * 64 * 16;
    return std::max(xb, red) + static_cast<size_t>(d.J + d.Jc) * 4;
}

template <int RB, int C_T, bool FROM_HASH>
ss1_status launch_split_cfg(const ForwardArgs& a, int Q, float* part) {
    const Dims& d = a.d;
    const size_t lds = split_lds(Q, d);
    auto kern = &split_kernel<RB, C_T, FROM_HASH>;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds)) != hipSuccess)
        return SS1_ERR_HIP;
    hipLaunchKernelGGL((split_kernel<RB, C_T, FROM_HASH>), dim3(static_cast<unsigned>(d.G * Q)),
                       dim3(kDecWaves * 64), lds, static_cast<hipStream_t>(a.stream),
                       static_cast<const uint16_t*>(a.x), static_cast<const uint16_t*>(a.w), a.plan_i, a.plan_s,
                       part, static_cast<int>(a.M), static_cast<int>(d.K), static_cast<int>(d.N),
                       static_cast<int>(d.J), static_cast<int>(d.Jc), d.c, d.BK, Q);
    if (hipGetLastError() != hipSuccess) return SS1_ERR_HIP;
    const long long quads = a.M * d.N / 4;
    hipLaunchKernelGGL(split_sum_kernel, dim3(static_cast<unsigned>((quads + 255) / 256)), dim3(256), 0,
                       static_cast<hipStream_t>(a.stream), part, static_cast<uint16_t*>(a.y),
                       static_cast<int>(a.M), static_cast<int>(d.N), Q, a.act);
    return hipGetLastError() == hipSuccess ? SS1_OK : SS1_ERR_HIP;
}

template <int RB, bool FROM_HASH>
ss1_status launch_split_rb(const ForwardArgs& a, int Q, float* part) {
    if (a.d.c == 2) return launch_split_cfg<RB, 2, FROM_HASH>(a, Q, part);
    return launch_split_cfg<RB, 0, FROM_HASH>(a, Q, part);
}

}  // namespace

// Slices per group of the column-split decode, or 0 when it does not apply:
// bf16, M <= 16, BN 32 or 64, BK % 64 == 0; the fewest slices Q (a power of
// two up to 16) that give at least one block per compute unit and whose
// staged rows fit in LDS, with K/Q a multiple of 512 (whole wave-wide loads
// per row) and Kc/Q a multiple of BK (whole compressed chunks per slice).
int split_slices(const ForwardArgs& a) {
    const Dims& d = a.d;
    if (a.dtype != SS1_BF16 || a.w_fp8 || a.M > 16 || a.M < 1) return 0;
    if ((d.BN != 32 && d.BN != 64) || d.BK % 64 != 0) return 0;
    if (d.J > kPlanPerThread * kDecWaves * 64) return 0;
    if (static_cast<double>(d.BN) * d.Kc * 2 >= 1073741824.0) return 0;
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    for (int Q = 1; Q <= 16; Q *= 2) {
        if (d.K % (512LL * Q) != 0 || d.Kc % (static_cast<long long>(d.BK) * Q) != 0) break;
        if (split_lds(Q, d) > static_cast<size_t>(max_lds())) continue;
        if (d.G * Q >= cus) return Q;
    }
    return 0;
}

size_t split_workspace_bytes(const ForwardArgs& a) {
    const int Q = split_slices(a);
    return Q > 0 ? static_cast<size_t>(Q) * a.M * a.d.N * 4 : 0;
}

ss1_status launch_split(const ForwardArgs& a, void* workspace) {
    const int Q = split_slices(a);
    if (Q == 0) return SS1_ERR_ALGO;
    float* part = static_cast<float*>(workspace);
    const bool hash = a.form == PlanForm::Hash;
    if (a.d.BN == 64) return hash ? launch_split_rb<4, true>(a, Q, part) : launch_split_rb<4, false>(a, Q, part);
    return hash ? launch_split_rb<2, true>(a, Q, part) : launch_split_rb<2, false>(a, Q, part);
}

bool decode_supported(const ForwardArgs& a) {
    const Dims& d = a.d;
    if (a.dtype != SS1_BF16 || a.w_fp8 || a.M > 16) return false;
    if (d.K % 512 != 0 || d.BK % 32 != 0 || (d.BN != 32 && d.BN != 64)) return false;
    if (d.J > kPlanPerThread * kDecWaves * 64) return false;
    if (static_cast<double>(d.BN) * d.Kc * 2 >= 2147483648.0) return false;
    return decode_lds(d.K, d) <= static_cast<size_t>(max_lds());
}

ss1_status launch_decode(const ForwardArgs& a) {
    const bool hash = a.form == PlanForm::Hash;
    if (a.d.BN == 64) return hash ? launch_decode_rb<4, true>(a) : launch_decode_rb<4, false>(a);
    return hash ? launch_decode_rb<2, true>(a) : launch_decode_rb<2, false>(a);
}

}  // namespace ss1
