// HIP kernels of the SS1 forward for gfx950 (CDNA4), and their launchers.
//
// The method ("SS1: Accelerating Inference with Fast and Expressive Sketch
// Structured Transform", summary page, "Approach"): sketch the layer input by
// signed additions of BK-wide input chunks into Kc = K/c compressed positions,
// one sketch per group of BN neurons, then contract each group's sketch with
// its BN rows of the compressed weight W_c.
//
// Kernels:
//   sketch_kernel   standalone sketch z[g][m][k'] (float32 sum, optional bf16).
//   generic_kernel  any dtype / chunking: per block a 64x64 output tile of one
//                   group, sketch slab and weight slab staged in LDS as
//                   float32, 4x4 register micro-tiles of fused multiply-adds.
//                   This is the exact float32 path.
//   fused_kernel    bf16, any M: per block an MT x BN tile of one group; every
//                   k-stage builds the sketched input tile in LDS from c
//                   coalesced chunk reads (float32 sum, then bf16), stages the
//                   W_c tile beside it, and runs 16x16x32 bf16 MFMA with
//                   float32 accumulators.  Double-buffered LDS, one barrier
//                   per stage, XCD-aware tile order.
//   smallm_kernel   bf16, M <= 16 (decode): per block 16 neurons of one group;
//                   its waves split Kc, build their 16x32 sketch fragments in
//                   registers straight from x and stream W_c once from HBM into
//                   MFMA operands; partial tiles are summed in LDS in a fixed
//                   order.
//
// Every kernel reads the plan of its group into LDS first, either from the
// forward hash/sign (inverting it there) or from the inverse index.  Source
// offsets are always built from a chunk number in [0, J), so no plan content
// can make a kernel read outside x.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>

#include "ss1_device.h"
#include "ss1_internal.h"
#include "ss1_msketch.h"

namespace ss1 {

namespace {

using namespace dev;

// ============================================================ sketch kernel
template <typename TIn, bool OUT_BF16, bool FROM_HASH>
__global__ __launch_bounds__(256) void sketch_kernel(const TIn* __restrict__ x,
                                                     const int32_t* __restrict__ pi,
                                                     const int8_t* __restrict__ ps,
                                                     void* __restrict__ z, int M, int K, int J,
                                                     int Jc, int c, int BK, int Kc) {
    extern __shared__ uint32_t smem[];
    uint32_t* s_src = smem;
    int* s_cnt = reinterpret_cast<int*>(smem + J);
    const int g = blockIdx.y;
    stage_plan<FROM_HASH>(pi, ps, g, J, Jc, c, BK, s_src, s_cnt);

    constexpr bool IN_BF16 = sizeof(TIn) == 2;
    constexpr int V = 16 / sizeof(TIn);  // elements per 16-byte vector
    const int vpc = BK / V;
    const long long items = static_cast<long long>(M) * Jc * vpc;
    const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
    for (long long it = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; it < items;
         it += stride) {
        const int v = static_cast<int>(it % vpc);
        const long long rest = it / vpc;
        const int t = static_cast<int>(rest % Jc);
        const int m = static_cast<int>(rest / Jc);
        const TIn* xr = x + static_cast<size_t>(m) * K + v * V;
        float acc[8];
        for (int r = 0; r < c; ++r) {
            const uint32_t e = s_src[t * c + r];
            const float s = entry_sign(e);
            const uint4 raw = *reinterpret_cast<const uint4*>(xr + (e & kOffMask));
            if constexpr (IN_BF16) {
                acc_bf16x8(acc, raw, s, r == 0);
            } else {
                const float f[4] = {__uint_as_float(raw.x), __uint_as_float(raw.y),
                                    __uint_as_float(raw.z), __uint_as_float(raw.w)};
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = (r == 0) ? s * f[i] : fmaf(s, f[i], acc[i]);
            }
        }
        const size_t o = (static_cast<size_t>(g) * M + m) * Kc + static_cast<size_t>(t) * BK + v * V;
        if constexpr (OUT_BF16) {
            static_assert(V == 8, "bf16 output needs bf16 input");
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(z) + o) = pack_bf16x8(acc);
        } else {
            float* zo = static_cast<float*>(z) + o;
            *reinterpret_cast<float4*>(zo) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            if constexpr (V == 8)
                *reinterpret_cast<float4*>(zo + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
        }
    }
}

// =========================================================== generic kernel
// Block: 256 threads as 16 x 16, output tile 64 rows x 64 columns of one group
// (columns [nt*64, nt*64+64) of the group, clipped to BN), 4 x 4 per thread.
// k' runs in ascending order; every product is a float32 fused multiply-add.
template <typename TIn, bool BF16_SKETCH_AND_OUT, bool FROM_HASH>
__global__ __launch_bounds__(256) void generic_kernel(const TIn* __restrict__ x,
                                                      const TIn* __restrict__ w,
                                                      const int32_t* __restrict__ pi,
                                                      const int8_t* __restrict__ ps,
                                                      void* __restrict__ y, int M, int K, int N,
                                                      int J, int Jc, int c, int BK, int BN,
                                                      int KW, int n_sub, int act) {
    constexpr int TM = 64, TN = 64, KWMAX = 32;
    __shared__ float zs[KWMAX][TM + 4];
    __shared__ float ws[KWMAX][TN + 4];
    extern __shared__ uint32_t smem[];
    uint32_t* s_src = smem;
    int* s_cnt = reinterpret_cast<int*>(smem + J);

    const int G = N / BN;
    const int sub = blockIdx.x % n_sub;
    const int g = (blockIdx.x / n_sub) % G;
    const int mt = blockIdx.x / (n_sub * G);
    stage_plan<FROM_HASH>(pi, ps, g, J, Jc, c, BK, s_src, s_cnt);

    const int m0 = mt * TM;
    const int col0 = sub * TN;                  // column inside the group
    const int width = min(TN, BN - col0);       // columns of this tile
    const int n0 = g * BN + col0;
    const int Kc = Jc * BK;
    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;

    auto load = [](const TIn* p) -> float {
        if constexpr (sizeof(TIn) == 2)
            return __uint_as_float(static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(p)) << 16);
        else
            return *reinterpret_cast<const float*>(p);
    };

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

    for (int t = 0; t < Jc; ++t) {
        for (int u0 = 0; u0 < BK; u0 += KW) {
            // sketch slab [TM][KW] and weight slab [TN][KW], stored k-major
            for (int e = tid; e < TM * KW; e += 256) {
                const int r = e / KW, k = e % KW;
                const int m = m0 + r;
                float v = 0.0f;
                if (m < M) {
                    const TIn* xr = x + static_cast<size_t>(m) * K + u0 + k;
                    for (int q = 0; q < c; ++q) {
                        const uint32_t en = s_src[t * c + q];
                        const float s = entry_sign(en);
                        const float xv = load(xr + (en & kOffMask));
                        v = (q == 0) ? s * xv : fmaf(s, xv, v);
                    }
                    if (BF16_SKETCH_AND_OUT) v = round_to_bf16(v);
                }
                zs[k][r] = v;
            }
            for (int e = tid; e < TN * KW; e += 256) {
                const int r = e / KW, k = e % KW;
                float v = 0.0f;
                if (r < width) v = load(w + static_cast<size_t>(n0 + r) * Kc + t * BK + u0 + k);
                ws[k][r] = v;
            }
            __syncthreads();
            for (int k = 0; k < KW; ++k) {
                float a[4], b[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = zs[k][ty * 4 + i];
#pragma unroll
                for (int j = 0; j < 4; ++j) b[j] = ws[k][tx * 4 + j];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
            }
            __syncthreads();
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty * 4 + i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int cc = tx * 4 + j;
            if (cc >= width) continue;
            const size_t o = static_cast<size_t>(m) * N + n0 + cc;
            if (BF16_SKETCH_AND_OUT)
                static_cast<uint16_t*>(y)[o] = to_bf16_bits(apply_act(acc[i][j], act));
            else
                static_cast<float*>(y)[o] = apply_act(acc[i][j], act);
        }
    }
}

// ============================================================= fused kernel
// Block: 256 threads (4 waves as WM x WN), output tile MT x BN of one group.
// Stage s covers k' in [s*KS, s*KS + KS), all inside compressed chunk
// t = s*KS / BK (KS divides BK).  LDS rows are padded by 8 bf16 (16 bytes).
// The sketch tile of a stage is summed in registers (sign flip + FMA, float32)
// and written to LDS as bf16 next to the W_c tile; both are double-buffered.
template <int MT, int BN, int WM, int WN, int KS, int C_T, bool W8, bool FROM_HASH>
__global__ __launch_bounds__(256) void fused_kernel(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ w,
                                                    const int32_t* __restrict__ pi,
                                                    const int8_t* __restrict__ ps,
                                                    uint16_t* __restrict__ y, int M, int K, int N,
                                                    int J, int Jc, int c_rt, int BK, int n_mt, int act,
                                                    const float* __restrict__ wscale) {
    static_assert(WM * WN == 4, "four waves");
    constexpr int TMW = MT / WM, TNW = BN / WN;  // wave tile
    constexpr int FM = TMW / 16, FN = TNW / 16;  // 16x16 MFMA blocks per wave
    static_assert(FM * 16 == TMW && FN * 16 == TNW, "wave tile must be a multiple of 16");
    constexpr int LDP = KS + 8;                  // LDS row pitch (elements)
    constexpr int VPR = KS / 8;                  // 16-byte vectors per tile row
    constexpr int AV = MT * VPR / 256;           // sketch vectors per thread per stage
    constexpr int BV = (BN * VPR + 255) / 256;   // weight vectors per thread per stage
    static_assert(AV * 256 == MT * VPR, "A tile must split evenly");
    constexpr int CR = (C_T > 0) ? C_T : 1;      // raw sources held per vector

    extern __shared__ uint32_t smem[];
    uint16_t* As = reinterpret_cast<uint16_t*>(smem);          // [2][MT][LDP]
    uint16_t* Bs = As + 2 * MT * LDP;                          // [2][BN][LDP]
    uint32_t* s_src = reinterpret_cast<uint32_t*>(Bs + 2 * BN * LDP);
    int* s_cnt = reinterpret_cast<int*>(s_src + J);

    const int c = (C_T > 0) ? C_T : c_rt;
    const int G = N / BN;
    // Tile order: each XCD works through a contiguous range of tiles (see
    // xcd_tile), and inside that range the two row tiles of a pair come
    // next to each other for every group, so the blocks running together on
    // one XCD share one pair of row bands (x gathers hit L2) and each W_c
    // slice they fetch serves two row tiles.
    constexpr int MG = 2;
    const int tile = xcd_tile(blockIdx.x, n_mt * G);
    const int mgi = tile / (MG * G);
    const int mg_eff = min(MG, n_mt - mgi * MG);
    const int rem = tile - mgi * MG * G;
    const int g = rem / mg_eff;
    const int mt = mgi * MG + rem % mg_eff;
    stage_plan<FROM_HASH>(pi, ps, g, J, Jc, c, BK, s_src, s_cnt);

    const int m0 = mt * MT;
    const int n0 = g * BN;
    const int Kc = Jc * BK;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int nstage = Kc / KS;

    // per-thread load coordinates; rows past M read row M-1 (never stored)
    int a_row[AV], a_col[AV];
    size_t a_src[AV];
#pragma unroll
    for (int i = 0; i < AV; ++i) {
        const int v = tid + i * 256;
        a_row[i] = v / VPR;
        a_col[i] = (v % VPR) * 8;
        a_src[i] = static_cast<size_t>(min(m0 + a_row[i], M - 1)) * K + a_col[i];
    }
    constexpr bool B_FULL = (BN * VPR) % 256 == 0;
    int b_row[BV], b_col[BV];
    bool b_ok[BV];
#pragma unroll
    for (int i = 0; i < BV; ++i) {
        const int v = tid + i * 256;
        b_row[i] = v / VPR;
        b_col[i] = (v % VPR) * 8;
        b_ok[i] = B_FULL || v < BN * VPR;
        if (!b_ok[i]) b_row[i] = 0;
    }

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int fr = lane & 15;       // row (A) / column (B) inside a 16x16 block
    const int fk = (lane >> 4) * 8; // first k of this lane's 8
    auto mma = [&](int buf) {
        const uint16_t* A = As + buf * MT * LDP;
        const uint16_t* B = Bs + buf * BN * LDP;
#pragma unroll
        for (int kk = 0; kk < KS; kk += 32) {
            bf16x8 af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(A + (wm * TMW + i * 16 + fr) * LDP + kk + fk);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(B + (wn * TNW + j * 16 + fr) * LDP + kk + fk);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    };

    if constexpr (C_T > 0) {
        // Register stage: the raw source vectors of the sketch tile, their
        // signs, and the W_c tile of one k-stage.  Stage s+2 is requested
        // while stage s is multiplied, and written to LDS (summed, rounded)
        // one stage later; the order is pinned with scheduling barriers.
        constexpr bool DEEP = C_T * AV <= 8;  // two register stages fit without spilling
        struct Regs {
            uint4 a[AV][CR];
            float sg[CR];
            uint32_t sx[CR];
            WRaw<W8> b[BV];
        };
        auto issue = [&](int s, Regs& R) {
            s = min(s, nstage - 1);
            const int k0 = s * KS;
            const int t = k0 / BK;
            const int u0 = k0 - t * BK;
#pragma unroll
            for (int r = 0; r < C_T; ++r) {
                const uint32_t e = __builtin_amdgcn_readfirstlane(s_src[t * C_T + r]);
                R.sg[r] = entry_sign(e);
                R.sx[r] = entry_sign_xor(e);
                const uint16_t* src = x + (e & kOffMask) + u0;
#pragma unroll
                for (int i = 0; i < AV; ++i) R.a[i][r] = *reinterpret_cast<const uint4*>(src + a_src[i]);
            }
#pragma unroll
            for (int i = 0; i < BV; ++i) R.b[i].load(w, static_cast<size_t>(n0 + b_row[i]) * Kc + k0 + b_col[i]);
        };
        auto commit = [&](const Regs& R, int buf) {
            uint16_t* A = As + buf * MT * LDP;
            uint16_t* B = Bs + buf * BN * LDP;
#pragma unroll
            for (int i = 0; i < AV; ++i) {
                uint4 v;
                if constexpr (C_T == 1) {
                    const uint32_t fl = R.sx[0];
                    v = make_uint4(R.a[i][0].x ^ fl, R.a[i][0].y ^ fl, R.a[i][0].z ^ fl, R.a[i][0].w ^ fl);
                } else {
                    float sum[8];
#pragma unroll
                    for (int r = 0; r < C_T; ++r) acc_sign8(sum, R.a[i][r], R.sg[r], R.sx[r], r == 0);
                    v = pack_bf16x8(sum);
                }
                *reinterpret_cast<uint4*>(A + a_row[i] * LDP + a_col[i]) = v;
            }
#pragma unroll
            for (int i = 0; i < BV; ++i)
                if (b_ok[i]) *reinterpret_cast<uint4*>(B + b_row[i] * LDP + b_col[i]) = R.b[i].bf16();
        };

        if constexpr (DEEP) {
            Regs r0, r1;
            issue(0, r0);
            issue(1, r1);
            commit(r0, 0);
            lds_barrier();
            int s = 0;
            for (; s + 2 <= nstage; s += 2) {
                issue(s + 2, r0);
                __builtin_amdgcn_sched_barrier(0);
                mma(0);
                __builtin_amdgcn_sched_barrier(0);
                commit(r1, 1);  // stage s+1 (re-writes the last stage when s+1 == nstage)
                lds_barrier();
                issue(s + 3, r1);
                __builtin_amdgcn_sched_barrier(0);
                mma(1);
                __builtin_amdgcn_sched_barrier(0);
                commit(r0, 0);  // stage s+2
                lds_barrier();
            }
            if (s < nstage) mma(0);
        } else {
            // one register stage: stage s+1 is requested while stage s is multiplied
            Regs r0;
            issue(0, r0);
            commit(r0, 0);
            lds_barrier();
            for (int s = 0; s < nstage; ++s) {
                issue(s + 1, r0);
                __builtin_amdgcn_sched_barrier(0);
                mma(s & 1);
                __builtin_amdgcn_sched_barrier(0);
                commit(r0, (s + 1) & 1);  // past the last stage this re-writes the idle buffer
                lds_barrier();
            }
        }
    } else {
        // runtime c: stage the sketch straight from global memory each step
        auto build = [&](int s, int buf) {
            const int k0 = s * KS;
            const int t = k0 / BK;
            const int u0 = k0 - t * BK;
            uint16_t* A = As + buf * MT * LDP;
            uint16_t* B = Bs + buf * BN * LDP;
#pragma unroll
            for (int i = 0; i < AV; ++i) {
                float sum[8];
                for (int r = 0; r < c; ++r) {
                    const uint32_t e = s_src[t * c + r];
                    const uint4 raw = *reinterpret_cast<const uint4*>(x + (e & kOffMask) + u0 + a_src[i]);
                    acc_sign8(sum, raw, entry_sign(e), entry_sign_xor(e), r == 0);
                }
                *reinterpret_cast<uint4*>(A + a_row[i] * LDP + a_col[i]) = pack_bf16x8(sum);
            }
#pragma unroll
            for (int i = 0; i < BV; ++i)
                if (b_ok[i]) {
                    WRaw<W8> r;
                    r.load(w, static_cast<size_t>(n0 + b_row[i]) * Kc + k0 + b_col[i]);
                    *reinterpret_cast<uint4*>(B + b_row[i] * LDP + b_col[i]) = r.bf16();
                }
        };
        build(0, 0);
        __syncthreads();
        for (int s = 0; s < nstage; ++s) {
            if (s + 1 < nstage) build(s + 1, (s + 1) & 1);
            mma(s & 1);
            __syncthreads();
        }
    }

    // epilogue: lane holds rows 4*(lane/16) + 0..3, column lane % 16 of each block
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * TNW + j * 16 + fr;
            const float ws = W8 ? wscale[col] : 1.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = m0 + wm * TMW + i * 16 + (lane >> 4) * 4 + q;
                if (m < M) y[static_cast<size_t>(m) * N + col] = to_bf16_bits(apply_act(acc[i][j][q] * ws, act));
            }
        }
    }
}

// ============================================================ small-M kernel
// Block: NW waves (4, 8 or 16, chosen from S and M), NB column blocks of 16
// neurons (rows nb*16*NB .. +16*NB-1 of group g).  Wave w takes the 32-wide
// k-steps [w*S/NW, (w+1)*S/NW) of the S = Kc/32 steps.  Per step each lane
// builds 8 sketch values of token (lane % 16) straight from x, once for all
// NB column blocks, and loads 8 weights of neuron (lane % 16) of each; one
// 16x16x32 MFMA per column block and step.  Tokens >= M are zero rows.
// BK % 32 == 0 keeps a step inside one compressed chunk.  W_c is read
// coalesced and permuted into the operand pattern across lanes.
template <int NW, int C_T, bool W8, bool FROM_HASH, int NB>
__global__ __launch_bounds__(NW * 64) void smallm_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ w,
                                                         const int32_t* __restrict__ pi,
                                                         const int8_t* __restrict__ ps,
                                                         uint16_t* __restrict__ y, int M, int K,
                                                         int N, int J, int Jc, int c_rt, int BK,
                                                         int BN, int act, const float* __restrict__ wscale) {
    extern __shared__ uint32_t smem[];
    f32x4* red = reinterpret_cast<f32x4*>(smem);                  // [NB][NW][64]
    uint32_t* s_src = smem + NB * NW * 64 * 4;
    int* s_cnt = reinterpret_cast<int*>(s_src + J);

    const int c = (C_T > 0) ? C_T : c_rt;
    const int nblk = BN / (16 * NB);
    const int g = blockIdx.x / nblk;
    const int nb = blockIdx.x % nblk;
    stage_plan<FROM_HASH>(pi, ps, g, J, Jc, c, BK, s_src, s_cnt);

    const int Kc = Jc * BK;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int S = Kc / 32;
    const int s_begin = static_cast<int>(static_cast<long long>(S) * wave / NW);
    const int s_end = static_cast<int>(static_cast<long long>(S) * (wave + 1) / NW);

    const int tok = lane & 15;
    const int kq = (lane >> 4) * 8;
    const bool tok_ok = tok < M;
    const uint16_t* xrow = x + static_cast<size_t>(tok_ok ? tok : 0) * K + kq;
    // W_c is read coalesced (this lane: neuron lane/4 of the block, k-chunk
    // lane%4) and permuted into the MFMA operand pattern before use
    // (column block b: the next 16 rows, 16 * Kc elements on)
    const int n = g * BN + nb * 16 * NB + (lane >> 2);
    const size_t wrow = static_cast<size_t>(n) * Kc + (lane & 3) * 8;  // element offset
    const size_t wblk = static_cast<size_t>(16) * Kc;
    const int perm_src = coalesced_src_lane_bytes(lane);

    f32x4 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    constexpr int U = 4;  // steps in flight per wave
    int s = s_begin;
    for (; s + U <= s_end; s += U) {
        WRaw<W8> wr[U][NB];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int b = 0; b < NB; ++b) wr[u][b].load(w, wrow + b * wblk + (s + u) * 32);
        uint4 xr[U][(C_T > 0) ? C_T : 1];
        float sg[U][(C_T > 0) ? C_T : 1];
        if constexpr (C_T > 0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k0 = (s + u) * 32;
                const int t = k0 / BK;
                const int u0 = k0 - t * BK;
#pragma unroll
                for (int r = 0; r < C_T; ++r) {
                    const uint32_t e = s_src[t * C_T + r];
                    sg[u][r] = entry_sign(e);
                    xr[u][r] = tok_ok ? *reinterpret_cast<const uint4*>(xrow + (e & kOffMask) + u0)
                                      : make_uint4(0, 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float a[8];
            if constexpr (C_T > 0) {
#pragma unroll
                for (int r = 0; r < C_T; ++r) acc_bf16x8(a, xr[u][r], sg[u][r], r == 0);
            } else {
                const int k0 = (s + u) * 32;
                const int t = k0 / BK;
                const int u0 = k0 - t * BK;
                for (int r = 0; r < c; ++r) {
                    const uint32_t e = s_src[t * c + r];
                    const uint4 raw = tok_ok ? *reinterpret_cast<const uint4*>(xrow + (e & kOffMask) + u0)
                                             : make_uint4(0, 0, 0, 0);
                    acc_bf16x8(a, raw, entry_sign(e), r == 0);
                }
            }
            const uint4 ap = pack_bf16x8(a);
#pragma unroll
            for (int b = 0; b < NB; ++b)
                acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, ap),
                    __builtin_bit_cast(bf16x8, to_operand_layout(wr[u][b].bf16(), perm_src)), acc[b], 0, 0, 0);
        }
    }
    for (; s < s_end; ++s) {
        WRaw<W8> wr[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) wr[b].load(w, wrow + b * wblk + s * 32);
        const int k0 = s * 32;
        const int t = k0 / BK;
        const int u0 = k0 - t * BK;
        float a[8];
        for (int r = 0; r < c; ++r) {
            const uint32_t e = s_src[t * c + r];
            const uint4 raw = tok_ok ? *reinterpret_cast<const uint4*>(xrow + (e & kOffMask) + u0)
                                     : make_uint4(0, 0, 0, 0);
            acc_bf16x8(a, raw, entry_sign(e), r == 0);
        }
        const uint4 ap = pack_bf16x8(a);
#pragma unroll
        for (int b = 0; b < NB; ++b)
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, ap), __builtin_bit_cast(bf16x8, to_operand_layout(wr[b].bf16(), perm_src)),
                acc[b], 0, 0, 0);
    }

#pragma unroll
    for (int b = 0; b < NB; ++b) red[(b * NW + wave) * 64 + lane] = acc[b];
    __syncthreads();
    // wave b < NB sums column block b over the waves
    if (wave < NB) {
        const f32x4* rb = red + wave * NW * 64;
        f32x4 sum = rb[lane];
        for (int v = 1; v < NW; ++v) {
            const f32x4 p = rb[v * 64 + lane];
            sum[0] += p[0];
            sum[1] += p[1];
            sum[2] += p[2];
            sum[3] += p[3];
        }
        const int col = g * BN + (nb * NB + wave) * 16 + (lane & 15);
        const float ws = W8 ? wscale[col] : 1.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int m = (lane >> 4) * 4 + q;
            if (m < M) y[static_cast<size_t>(m) * N + col] = to_bf16_bits(apply_act(sum[q] * ws, act));
        }
    }
}

// ============================================================== band kernel
// For layers whose input rows are short enough that a band of MT rows fits in
// LDS (MT*K bf16).  Block: NW waves; it loads input rows [m0, m0+MT) once and
// then each wave takes whole groups of the block's group range, one after
// another, with no further barrier.  Per 32-wide k-step a wave loads its
// group's W_c slice from global memory and, for each 16-row block of the band,
// reads the c source chunks from the band, sums them in float32 (sign flips
// and fused multiply-adds), rounds the sketch to bf16 and feeds it to one MFMA
// per 16 neurons.  The steps run as a two-stage software pipeline: the plan
// entries, band reads and W_c loads of step s+1 are issued before the
// arithmetic of step s, so LDS and L2 latency overlap with the math; the
// pipeline runs on across the wave's groups.
// The MFMA computes the transposed tile y^T = W_c * z^T so that each lane ends
// up with 4*BN/16 consecutive outputs of one row (W_c rows are loaded in the
// matching permuted order) and stores them as 16-byte vectors.
template <int MT, int BN, int C_T, int NW, int RS, int KH, bool RAW_PF, int PD, bool FROM_HASH, bool W8>
__global__ __launch_bounds__(NW * 64) void band_kernel(const uint16_t* __restrict__ x,
                                                       const uint16_t* __restrict__ w,
                                                       const int32_t* __restrict__ pi,
                                                       const int8_t* __restrict__ ps,
                                                       uint16_t* __restrict__ y, int M, int K, int N,
                                                       int J, int Jc, int c_rt, int BK, int gsplit, int act,
                                                       const float* __restrict__ wscale) {
    constexpr int RB = MT / 16;  // 16-row blocks of the band
    constexpr int NB = BN / 16;  // 16-neuron blocks of a group
    static_assert(RB * 16 == MT && NB * 16 == BN && NB % 2 == 0, "tile sizes");
    static_assert(KH == 1 || (KH == 2 && C_T > 0), "a step is 32*KH wide; 64 needs a fixed c");
    static_assert(!W8 || C_T > 0, "E4M3 weights with a fixed c");
    // weights: bf16, or E4M3 codes (one byte each) with one float32 scale per row
    constexpr int WB = W8 ? 1 : 2;
    using WV = typename std::conditional<W8, uint2, uint4>::type;
    // RS waves share a group, each taking RBW of the band's row blocks; NG
    // groups are in progress at a time
    constexpr int RBW = RB / RS;
    constexpr int NG = NW / RS;
    static_assert(RBW * RS == RB && NG * RS == NW, "row split");
    constexpr int CR = (C_T > 0) ? C_T : 1;
    extern __shared__ uint32_t smem[];
    const int LDK = K + 8;  // band row pitch (elements): 16-byte skew between rows
    uint16_t* band = reinterpret_cast<uint16_t*>(smem);
    uint32_t* s_src = smem + (MT * LDK) / 2;

    const int c = (C_T > 0) ? C_T : c_rt;
    const int G = N / BN;
    const int bi = blockIdx.x / gsplit;
    const int gs = blockIdx.x - bi * gsplit;
    const int g0 = static_cast<int>(static_cast<long long>(G) * gs / gsplit);
    const int g1 = static_cast<int>(static_cast<long long>(G) * (gs + 1) / gsplit);
    const int GW = g1 - g0;
    int* s_cnt = reinterpret_cast<int*>(s_src + GW * J);
    const int m0 = bi * MT;

    // band of input rows, zero rows past M; eight 16-byte loads in flight per
    // thread before their LDS stores
    {
        constexpr int U = 8;
        const int vpr = K / 8;
        const int total = MT * vpr;
        for (int v0 = threadIdx.x; v0 < total; v0 += U * NW * 64) {
            uint4 val[U];
            int dst[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = v0 + u * NW * 64;
                const int r = v / vpr;
                const int col = (v - r * vpr) * 8;
                dst[u] = (v < total) ? r * LDK + col : -1;
                val[u] = make_uint4(0, 0, 0, 0);
                if (v < total && m0 + r < M)
                    val[u] = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(m0 + r) * K + col);
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (dst[u] >= 0) *reinterpret_cast<uint4*>(band + dst[u]) = val[u];
        }
    }
    stage_plans<FROM_HASH>(pi, ps, g0, GW, J, Jc, c, BK, s_src, s_cnt);  // ends with a barrier

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar addressing
    const int gl0 = wave / RS;          // first group (inside the block's range) of this wave
    const int rb0 = (wave % RS) * RBW;  // first row block of this wave
    const int li = lane & 15;          // MFMA row/column index of this lane
    const int q = lane >> 4;           // which 8 of the 32 k of a step, and output quarter
    const int Kc = Jc * BK;
    const int steps = Kc / (32 * KH);  // KH == 2 needs BK % 64 == 0 (a step stays in one chunk)
    // MFMA row r of neuron block nb is neuron (r/4)*4*NB + nb*4 + r%4 of the
    // group.  W_c is loaded coalesced (this lane: row lane/4 of the block,
    // k-chunk lane%4) and permuted into the operand pattern before use.
    // (byte offsets inside the group's W_c slice; BN*Kc*2 is far below 2^32
    // for any layer whose band fits in LDS)
    uint32_t woff[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int r = lane >> 2;
        woff[nb] = static_cast<uint32_t>(((r >> 2) * 4 * NB + nb * 4 + (r & 3)) * Kc + (lane & 3) * 8) * WB;
    }
    const uint32_t wslice_bytes = static_cast<uint32_t>(BN * Kc * WB);
    const uint8_t* wbytes = reinterpret_cast<const uint8_t*>(w);
    const int perm_src = coalesced_src_lane_bytes(lane);
    const uint16_t* lrow = band + (rb0 * 16 + li) * LDK + q * 8;  // this lane's band row (first block), k offset
    // c = 2, 4, 8: the sketch runs on the matrix cores (see compute); each
    // lane reads 16 inputs of one source per pair, at 16*(q%2) of a 32-wide
    // half-step.  Other c keep the float32 sketch on the vector ALUs.
    constexpr bool MSK = C_T == 2 || C_T == 4 || C_T == 8;
    const uint16_t* lrow_ms = band + (rb0 * 16 + li) * LDK + 16 * (q & 1);
    uint4 sel_one, sel_neg;
    sketch_selector_base(li, q, sel_one, sel_neg);

    // lane holds y[m0 + (rb0+rb)*16 + li][g*BN + q*4*NB + nb*4 + i] of acc[rb][nb][i]
    auto store_tile = [&](int g, f32x4 (&acc)[RBW][NB]) {
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
            const int m = m0 + (rb0 + rb) * 16 + li;
            if (m >= M) continue;
            uint16_t* yr = y + static_cast<size_t>(m) * N + static_cast<size_t>(g) * BN + q * 4 * NB;
            if constexpr (W8) {  // the rows' E4M3 scales (neuron g*BN + q*4*NB + nb*4 + i)
                const float* sc = wscale + static_cast<size_t>(g) * BN + q * 4 * NB;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[rb][nb][i] *= sc[nb * 4 + i];
            }
#pragma unroll
            for (int h = 0; h < NB / 2; ++h) {
                uint4 o;
                o.x = pack_bf16(apply_act(acc[rb][2 * h][0], act), apply_act(acc[rb][2 * h][1], act));
                o.y = pack_bf16(apply_act(acc[rb][2 * h][2], act), apply_act(acc[rb][2 * h][3], act));
                o.z = pack_bf16(apply_act(acc[rb][2 * h + 1][0], act), apply_act(acc[rb][2 * h + 1][1], act));
                o.w = pack_bf16(apply_act(acc[rb][2 * h + 1][2], act), apply_act(acc[rb][2 * h + 1][3], act));
                *reinterpret_cast<uint4*>(yr + h * 8) = o;
            }
        }
#pragma unroll
        for (int i = 0; i < RBW; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    };

    f32x4 acc[RBW][NB];
#pragma unroll
    for (int i = 0; i < RBW; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    if constexpr (C_T > 0) {
        // Two-stage software pipeline over the wave's (group, step) items:
        // the operands of the next item (the next group's first step at a
        // group's end) are requested before the arithmetic of the current
        // one.  Every prefetch is unconditional (past the last item it
        // re-reads the last one) and the order is pinned with scheduling
        // barriers, so the compiler neither sinks a prefetch next to its use
        // nor has to wait conservatively at control-flow joins; a group's
        // output stores come after the prefetch of the next group.
        const int ngw = (gl0 < GW) ? (GW - gl0 + NG - 1) / NG : 0;
        // A stage holds what one step needs from outside LDS: its W_c slices
        // (prefetched a step ahead) and its plan entries.  With RAW_PF the band
        // reads are prefetched too; otherwise they are issued at the start of
        // the step, ahead of the operand permutes.
        struct Stage {
            WV wf[KH][NB];
            float sg[CR];
            uint32_t sx[CR];
            uint32_t off[CR];
            uint4 raw[RAW_PF ? KH : 1][RAW_PF ? RBW : 1][RAW_PF ? CR : 1];
        };
        auto read_band = [&](const Stage& st, uint4 (&raw)[KH][RBW][CR]) {
            if constexpr (MSK) {
                // source pair p: lanes 0-31 read source 2p, lanes 32-63 source
                // 2p+1, 16 consecutive inputs at 16*(q%2) of each 32-wide half
#pragma unroll
                for (int p = 0; p < C_T / 2; ++p) {
                    // select between the two values, not the two array elements: a
                    // lane-dependent index puts the whole stage in scratch memory
                    const uint32_t o0 = __builtin_amdgcn_readfirstlane(st.off[2 * p]);
                    const uint32_t o1 = __builtin_amdgcn_readfirstlane(st.off[2 * p + 1]);
                    const uint16_t* src = lrow_ms + (q < 2 ? o0 : o1);
#pragma unroll
                    for (int h = 0; h < KH; ++h)
#pragma unroll
                        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
                            for (int e = 0; e < 2; ++e)
                                raw[h][rb][2 * p + e] =
                                    *reinterpret_cast<const uint4*>(src + rb * 16 * LDK + 32 * h + 8 * e);
                }
            } else {
#pragma unroll
                for (int r = 0; r < C_T; ++r) {
                    const uint16_t* src = lrow + st.off[r];
#pragma unroll
                    for (int h = 0; h < KH; ++h)
#pragma unroll
                        for (int rb = 0; rb < RBW; ++rb)
                            raw[h][rb][r] = *reinterpret_cast<const uint4*>(src + rb * 16 * LDK + 32 * h);
                }
            }
        };
        auto load = [&](int gi, int s, Stage& st) {
            if (gi >= ngw) {  // past the wave's last item: request the last one again
                gi = ngw - 1;
                s = steps - 1;
            }
            gi = __builtin_amdgcn_readfirstlane(gi);
            s = __builtin_amdgcn_readfirstlane(s);
            const int gl = gl0 + gi * NG;
            const uint32_t* plan = s_src + gl * J;
            const int k0 = s * 32 * KH;
            const int t = k0 / BK;
            const int ub = k0 - t * BK;
            // both 32-wide halves of a row's 128-byte line are requested back to back
            const auto wr = make_rsrc(wbytes + static_cast<size_t>(g0 + gl) * BN * Kc * WB, wslice_bytes);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int h = 0; h < KH; ++h) {
                    if constexpr (W8) {
                        st.wf[h][nb] = __builtin_bit_cast(
                            uint2, __builtin_amdgcn_raw_buffer_load_b64(wr, woff[nb], (k0 + 32 * h) * WB, 0));
                    } else {
                        st.wf[h][nb] = buf_load16(wr, woff[nb], (k0 + 32 * h) * 2);
                    }
                }
#pragma unroll
            for (int r = 0; r < C_T; ++r) {
                const uint32_t e = __builtin_amdgcn_readfirstlane(plan[t * C_T + r]);
                st.sg[r] = entry_sign(e);
                st.sx[r] = entry_sign_xor(e);
                st.off[r] = (e & kOffMask) + ub;
            }
            if constexpr (RAW_PF) read_band(st, st.raw);
        };
        auto compute = [&](const Stage& st) {
            uint4 rawj[KH][RBW][CR];
            if constexpr (!RAW_PF) read_band(st, rawj);
            const auto& raw = [&]() -> const uint4(&)[KH][RBW][CR] {
                if constexpr (RAW_PF) return st.raw; else return rawj;
            }();
#pragma unroll
            for (int h = 0; h < KH; ++h) {
                uint4 wop[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    if constexpr (W8) {
                        wop[nb] = to_operand_layout(fp8x8_to_bf16x8(st.wf[h][nb]), perm_src);
                    } else {
                        wop[nb] = to_operand_layout(st.wf[h][nb], perm_src);
                    }
                }
                if constexpr (MSK) {
                    // Sketch on the matrix cores: D[i][token] = sum_k A[i][k] X[k][token]
                    // with X this lane's 16 inputs of its source (k = 8q + e) and
                    // A the signed one-hot selection (sketch_selector).  Two
                    // MFMAs per source pair give the sketch columns 8q..8q+3 and
                    // 8q+4..8q+7 of the half-step for this lane's token, which is
                    // the contraction's operand layout; further pairs accumulate
                    // on the float32 result.  A pair adds exactly two signed bf16
                    // values (the other products are zeros), so at c = 2 the
                    // float32 result is the one rounding of the exact sum, as in
                    // the ascending float32 sketch; for c >= 4 the pairs' sums
                    // are added in pair order.
                    uint4 sel[C_T / 2];
#pragma unroll
                    for (int p = 0; p < C_T / 2; ++p) {
                        const uint32_t x0 = __builtin_amdgcn_readfirstlane(st.sx[2 * p]);
                        const uint32_t x1 = __builtin_amdgcn_readfirstlane(st.sx[2 * p + 1]);
                        const float g0 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                                       __builtin_bit_cast(int, st.sg[2 * p])));
                        const float g1 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                                       __builtin_bit_cast(int, st.sg[2 * p + 1])));
                        sel[p] = sketch_selector(sel_one, sel_neg, q < 2 ? x0 : x1, q < 2 ? g0 : g1);
                    }
                    f32x4 d0[RBW], d1[RBW];
#pragma unroll
                    for (int rb = 0; rb < RBW; ++rb) {
                        d0[rb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                        d1[rb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                        for (int p = 0; p < C_T / 2; ++p) {
                            const uint4 ra = raw[h][rb][2 * p], rbv = raw[h][rb][2 * p + 1];
                            const uint4 x0 = make_uint4(ra.x, ra.y, rbv.x, rbv.y);
                            const uint4 x1 = make_uint4(ra.z, ra.w, rbv.z, rbv.w);
                            d0[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, sel[p]), __builtin_bit_cast(bf16x8, x0), d0[rb], 0, 0, 0);
                            d1[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, sel[p]), __builtin_bit_cast(bf16x8, x1), d1[rb], 0, 0, 0);
                        }
                    }
#pragma unroll
                    for (int rb = 0; rb < RBW; ++rb) {
                        uint4 zp;
                        zp.x = pack_bf16(d0[rb][0], d0[rb][1]);
                        zp.y = pack_bf16(d0[rb][2], d0[rb][3]);
                        zp.z = pack_bf16(d1[rb][0], d1[rb][1]);
                        zp.w = pack_bf16(d1[rb][2], d1[rb][3]);
                        const bf16x8 zf = __builtin_bit_cast(bf16x8, zp);
                        __builtin_amdgcn_s_setprio(1);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, wop[nb]), zf, acc[rb][nb], 0, 0, 0);
                        __builtin_amdgcn_s_setprio(0);
                    }
                    continue;
                }
#pragma unroll
                for (int rb = 0; rb < RBW; ++rb) {
                    float a[8];
#pragma unroll
                    for (int r = 0; r < C_T; ++r) acc_sign8(a, raw[h][rb][r], st.sg[r], st.sx[r], r == 0);
                    const bf16x8 zf = __builtin_bit_cast(bf16x8, pack_bf16x8(a));
                    // raised issue priority over the row block's MFMAs (measured
                    // about 1% on GPT-2 S, and 5% in the backward fold kernels)
                    __builtin_amdgcn_s_setprio(1);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, wop[nb]), zf, acc[rb][nb], 0, 0, 0);
                    __builtin_amdgcn_s_setprio(0);
                }
            }
        };
        // Flat walk over the wave's (group, step) items with a ring of PD
        // stages: item i+PD-1 is requested before item i is computed.  The
        // item count is padded to a multiple of PD; padding items re-read the
        // last item and only touch accumulators that are never stored again.
        if (ngw > 0) {
            auto advance = [&](int& gi, int& s) {
                if (++s == steps) {
                    s = 0;
                    ++gi;
                }
            };
            const int total = ngw * steps;
            Stage st[PD];
            int lg = 0, ls = 0;  // next item to request
#pragma unroll
            for (int j = 0; j < PD - 1; ++j) {
                load(lg, ls, st[j]);
                advance(lg, ls);
            }
            int cg = 0, cs = 0;  // next item to compute
            for (int i0 = 0; i0 < total; i0 += PD) {
#pragma unroll
                for (int j = 0; j < PD; ++j) {
                    load(lg, ls, st[(j + PD - 1) % PD]);
                    advance(lg, ls);
                    __builtin_amdgcn_sched_barrier(0);
                    compute(st[j]);
                    __builtin_amdgcn_sched_barrier(0);
                    if (cs == steps - 1 && cg < ngw) store_tile(g0 + gl0 + cg * NG, acc);
                    advance(cg, cs);
                }
            }
        }
    } else {
        // runtime c: no pipelining
        for (int gl = gl0; gl < GW; gl += NG) {
            const int g = g0 + gl;
            const uint32_t* plan = s_src + gl * J;
            for (int s = 0; s < steps; ++s) {
                const int k0 = s * 32;
                const int t = k0 / BK;
                const int ub = k0 - t * BK;
                const auto wr = make_rsrc(w + static_cast<size_t>(g) * BN * Kc, wslice_bytes);
                uint4 wf[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) wf[nb] = to_operand_layout(buf_load16(wr, woff[nb], k0 * 2), perm_src);
#pragma unroll
                for (int rb = 0; rb < RBW; ++rb) {
                    float a[8];
                    for (int r = 0; r < c; ++r) {
                        const uint32_t e = __builtin_amdgcn_readfirstlane(plan[t * c + r]);
                        const uint4 raw = *reinterpret_cast<const uint4*>(lrow + rb * 16 * LDK + (e & kOffMask) + ub);
                        acc_sign8(a, raw, entry_sign(e), entry_sign_xor(e), r == 0);
                    }
                    const bf16x8 zf = __builtin_bit_cast(bf16x8, pack_bf16x8(a));
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, wf[nb]), zf, acc[rb][nb], 0, 0, 0);
                }
            }
            store_tile(g, acc);
        }
    }
}

// ================================================================ launchers
inline ss1_status launch_status() {
    return hipGetLastError() == hipSuccess ? SS1_OK : SS1_ERR_HIP;
}

// Small-M column blocks per block where the grid stays large enough (1 or 2).
constexpr int kSmallmPair = 2;

inline size_t plan_lds_bytes(const Dims& d) {
    return static_cast<size_t>(d.J) * 4 + static_cast<size_t>(d.Jc) * 4;
}

template <bool FROM_HASH>
ss1_status launch_generic_t(const ForwardArgs& a) {
    const Dims& d = a.d;
    int KW = 32;
    while (d.BK % KW) KW >>= 1;
    const int n_sub = static_cast<int>((d.BN + 63) / 64);
    const long long mt = (a.M + 63) / 64;
    const long long blocks = mt * d.G * n_sub;
    if (blocks > 0x7FFFFFFFLL) return SS1_ERR_SHAPE;
    hipStream_t st = static_cast<hipStream_t>(a.stream);
    const size_t lds = plan_lds_bytes(d);
    if (a.dtype == SS1_F32) {
        hipLaunchKernelGGL((generic_kernel<float, false, FROM_HASH>), dim3(static_cast<unsigned>(blocks)),
                           dim3(256), lds, st, static_cast<const float*>(a.x),
                           static_cast<const float*>(a.w), a.plan_i, a.plan_s, a.y, (int)a.M,
                           (int)d.K, (int)d.N, (int)d.J, (int)d.Jc, d.c, d.BK, d.BN, KW, n_sub, a.act);
    } else {
        hipLaunchKernelGGL((generic_kernel<uint16_t, true, FROM_HASH>), dim3(static_cast<unsigned>(blocks)),
                           dim3(256), lds, st, static_cast<const uint16_t*>(a.x),
                           static_cast<const uint16_t*>(a.w), a.plan_i, a.plan_s, a.y, (int)a.M,
                           (int)d.K, (int)d.N, (int)d.J, (int)d.Jc, d.c, d.BK, d.BN, KW, n_sub, a.act);
    }
    return launch_status();
}

template <int MT, int BN, int WM, int WN, int KS, int C_T, bool W8, bool FROM_HASH>
ss1_status launch_fused_cfg(const ForwardArgs& a) {
    const Dims& d = a.d;
    const int n_mt = static_cast<int>((a.M + MT - 1) / MT);
    const long long blocks = static_cast<long long>(n_mt) * d.G;
    if (blocks > 0x7FFFFFFFLL) return SS1_ERR_SHAPE;
    constexpr int LDP = KS + 8;
    const size_t lds = static_cast<size_t>(2) * (MT + BN) * LDP * 2 + plan_lds_bytes(d);
    auto kern = &fused_kernel<MT, BN, WM, WN, KS, C_T, W8, FROM_HASH>;
    if (lds > 64 * 1024) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                static_cast<int>(lds)) != hipSuccess)
            return SS1_ERR_HIP;
    }
    hipLaunchKernelGGL((fused_kernel<MT, BN, WM, WN, KS, C_T, W8, FROM_HASH>), dim3(static_cast<unsigned>(blocks)),
                       dim3(256), lds, static_cast<hipStream_t>(a.stream), static_cast<const uint16_t*>(a.x),
                       static_cast<const uint16_t*>(a.w), a.plan_i, a.plan_s, static_cast<uint16_t*>(a.y),
                       (int)a.M, (int)d.K, (int)d.N, (int)d.J, (int)d.Jc, d.c, d.BK, n_mt, a.act, a.wscale);
    return launch_status();
}

template <int BN, int WM, int WN, int KS, bool W8, bool FROM_HASH>
ss1_status launch_fused_c(const ForwardArgs& a) {
    switch (a.d.c) {
        case 1: return launch_fused_cfg<128, BN, WM, WN, KS, 1, W8, FROM_HASH>(a);
        case 2: return launch_fused_cfg<128, BN, WM, WN, KS, 2, W8, FROM_HASH>(a);
        case 4: return launch_fused_cfg<128, BN, WM, WN, KS, 4, W8, FROM_HASH>(a);
        case 8: return launch_fused_cfg<128, BN, WM, WN, KS, 8, W8, FROM_HASH>(a);
        default: return launch_fused_cfg<128, BN, WM, WN, KS, 0, W8, FROM_HASH>(a);
    }
}

template <int KS, bool W8, bool FROM_HASH>
ss1_status launch_fused_bn(const ForwardArgs& a) {
    switch (a.d.BN) {
        case 32: return launch_fused_c<32, 4, 1, KS, W8, FROM_HASH>(a);
        case 64: return launch_fused_c<64, 2, 2, KS, W8, FROM_HASH>(a);
        case 128: return launch_fused_c<128, 2, 2, KS, W8, FROM_HASH>(a);
        default: return SS1_ERR_ALGO;
    }
}

template <bool W8, bool FROM_HASH>
ss1_status launch_fused_t(const ForwardArgs& a) {
    if (a.d.BK % 64 == 0) return launch_fused_bn<64, W8, FROM_HASH>(a);
    return launch_fused_bn<32, W8, FROM_HASH>(a);
}

// Column blocks per small-M block: two 16-neuron blocks share each wave's
// sketch where that still leaves 1.5 blocks per compute unit.
inline int smallm_nb(const ForwardArgs& a) {
    return (a.d.BN % 32 == 0 && a.d.N / 32 >= 384) ? kSmallmPair : 1;
}

template <int NW, int C_T, bool W8, bool FROM_HASH, int NB>
ss1_status launch_smallm_cfg_nb(const ForwardArgs& a) {
    const Dims& d = a.d;
    const long long blocks = d.G * (d.BN / (16 * NB));
    if (blocks > 0x7FFFFFFFLL) return SS1_ERR_SHAPE;
    const size_t lds = static_cast<size_t>(NB) * NW * 64 * 16 + plan_lds_bytes(d);
    hipLaunchKernelGGL((smallm_kernel<NW, C_T, W8, FROM_HASH, NB>), dim3(static_cast<unsigned>(blocks)),
                       dim3(NW * 64), lds, static_cast<hipStream_t>(a.stream),
                       static_cast<const uint16_t*>(a.x), static_cast<const uint16_t*>(a.w),
                       a.plan_i, a.plan_s, static_cast<uint16_t*>(a.y), (int)a.M, (int)d.K,
                       (int)d.N, (int)d.J, (int)d.Jc, d.c, d.BK, d.BN, a.act, a.wscale);
    return launch_status();
}

template <int NW, int C_T, bool W8, bool FROM_HASH>
ss1_status launch_smallm_cfg(const ForwardArgs& a) {
    if (smallm_nb(a) == 2) return launch_smallm_cfg_nb<NW, C_T, W8, FROM_HASH, 2>(a);
    return launch_smallm_cfg_nb<NW, C_T, W8, FROM_HASH, 1>(a);
}

// Waves per block: about 16 of the Kc/32 k-steps per wave (measured on the
// Llama-3-8B decode shapes: 64 steps -> 4 waves best, 224 steps -> 16 waves at
// M = 1 but 8 at M = 16, where each step also reads 16 tokens); 16 waves only
// where the kernel fits in 128 registers (c <= 2).
template <int C_T, bool W8, bool FROM_HASH>
ss1_status launch_smallm_nw(const ForwardArgs& a) {
    const long long S = a.d.Kc / 32;
    if constexpr (C_T > 0 && C_T <= 2) {
        if (S >= 192 && a.M <= 8) return launch_smallm_cfg<16, C_T, W8, FROM_HASH>(a);
    }
    if (S >= 96) return launch_smallm_cfg<8, C_T, W8, FROM_HASH>(a);
    return launch_smallm_cfg<4, C_T, W8, FROM_HASH>(a);
}

template <bool W8, bool FROM_HASH>
ss1_status launch_smallm_t(const ForwardArgs& a) {
    switch (a.d.c) {
        case 1: return launch_smallm_nw<1, W8, FROM_HASH>(a);
        case 2: return launch_smallm_nw<2, W8, FROM_HASH>(a);
        case 4: return launch_smallm_nw<4, W8, FROM_HASH>(a);
        case 8: return launch_smallm_nw<8, W8, FROM_HASH>(a);
        default: return launch_smallm_nw<0, W8, FROM_HASH>(a);
    }
}

// ------------------------------------------------------------ band launch
struct DeviceInfo {
    int cus;
    int lds_per_block;
};

// Compute units and the largest LDS a block may take on the current device.
inline DeviceInfo device_info() {
    int dev = 0;
    DeviceInfo di{256, 64 * 1024};
    if (hipGetDevice(&dev) != hipSuccess) return di;
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) di.cus = v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && v > 0)
        di.lds_per_block = v;
    return di;
}

struct BandCfg {
    int MT;      // rows per band, 0 when the layer does not fit
    int gsplit;  // blocks per band, each taking a contiguous range of groups
    size_t lds;
};

inline size_t band_lds(int MT, const Dims& d, int gsplit) {
    const long long gw = (d.G + gsplit - 1) / gsplit;
    return static_cast<size_t>(MT) * (d.K + 8) * 2 + static_cast<size_t>(gw) * (d.J + d.Jc) * 4;
}

// Largest band (64, 48 or 32 rows) that fits in LDS, and the group split that
// gives every compute unit work while the group plans still fit.
inline BandCfg band_config(const Dims& d, int64_t M, const DeviceInfo& di) {
    for (int MT : {64, 48, 32}) {
        const long long nbands = (M + MT - 1) / MT;
        const size_t band_bytes = static_cast<size_t>(MT) * (d.K + 8) * 2;
        if (band_bytes + static_cast<size_t>(d.J + d.Jc) * 4 > static_cast<size_t>(di.lds_per_block)) continue;
        const long long per_cu = std::max<long long>(1, di.lds_per_block / static_cast<long long>(band_bytes + 1024));
        long long gsplit = (static_cast<long long>(di.cus) * per_cu + nbands - 1) / nbands;
        gsplit = std::max<long long>(1, std::min<long long>(gsplit, d.G));
        while (gsplit < d.G && band_lds(MT, d, static_cast<int>(gsplit)) > static_cast<size_t>(di.lds_per_block))
            ++gsplit;
        if (band_lds(MT, d, static_cast<int>(gsplit)) > static_cast<size_t>(di.lds_per_block)) continue;
        if (nbands * gsplit > 0x7FFFFFFFLL) continue;
        return BandCfg{MT, static_cast<int>(gsplit), band_lds(MT, d, static_cast<int>(gsplit))};
    }
    return BandCfg{0, 0, 0};
}

// Launch shapes of the band kernel:
//   WIDE (c <= 2, or c = 4 with BN <= 64; BK % 64 == 0): 64-wide steps, so each pair of W_c requests
//        covers whole 128-byte lines; band reads issued at the start of a step
//   BASE: 32-wide steps, band reads a step ahead where registers allow
// Both run 8 waves (4 when the tile needs more than 256 registers) with W_c
// requested one step ahead.  (Splitting a group's rows over two waves for
// four waves per SIMD measured slower: the kernel is not latency-starved.)
enum class BandShape { BASE, WIDE };

template <int MT, int BN, int C_T, BandShape SH, bool FROM_HASH, bool W8>
ss1_status launch_band_cfg(const ForwardArgs& a, const BandCfg& cfg) {
    const Dims& d = a.d;
    constexpr int NW = (BN == 128 || C_T >= 8 || (C_T == 4 && MT == 64)) ? 4 : 8;
    constexpr int RS = 1;
    constexpr int KH = SH == BandShape::WIDE ? 2 : 1;
    // (not with the matrix-core sketch of c = 2 and 4: its lane-dependent
    // source choice then kept the prefetched stage in scratch memory)
    constexpr bool RAW_PF = KH == 1 && C_T <= 4 && BN < 128 && C_T != 2 && C_T != 4;
    constexpr int PD = 2;
    const long long nbands = (a.M + MT - 1) / MT;
    auto kern = &band_kernel<MT, BN, C_T, NW, RS, KH, RAW_PF, PD, FROM_HASH, W8>;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(cfg.lds)) != hipSuccess)
        return SS1_ERR_HIP;
    hipLaunchKernelGGL((band_kernel<MT, BN, C_T, NW, RS, KH, RAW_PF, PD, FROM_HASH, W8>),
                       dim3(static_cast<unsigned>(nbands * cfg.gsplit)), dim3(NW * 64), cfg.lds,
                       static_cast<hipStream_t>(a.stream), static_cast<const uint16_t*>(a.x),
                       static_cast<const uint16_t*>(a.w), a.plan_i, a.plan_s, static_cast<uint16_t*>(a.y),
                       (int)a.M, (int)d.K, (int)d.N, (int)d.J, (int)d.Jc, d.c, d.BK, cfg.gsplit, a.act, a.wscale);
    return launch_status();
}

template <int MT, int BN, bool FROM_HASH, bool W8>
ss1_status launch_band_c(const ForwardArgs& a, const BandCfg& cfg) {
    const bool wide = a.d.BK % 64 == 0;
    switch (a.d.c) {
        case 1: return wide ? launch_band_cfg<MT, BN, 1, BandShape::WIDE, FROM_HASH, W8>(a, cfg)
                            : launch_band_cfg<MT, BN, 1, BandShape::BASE, FROM_HASH, W8>(a, cfg);
        case 2: return wide ? launch_band_cfg<MT, BN, 2, BandShape::WIDE, FROM_HASH, W8>(a, cfg)
                            : launch_band_cfg<MT, BN, 2, BandShape::BASE, FROM_HASH, W8>(a, cfg);
        case 4:
            if constexpr (BN <= 64)
                if (wide) return launch_band_cfg<MT, BN, 4, BandShape::WIDE, FROM_HASH, W8>(a, cfg);
            return launch_band_cfg<MT, BN, 4, BandShape::BASE, FROM_HASH, W8>(a, cfg);
        case 8: return launch_band_cfg<MT, BN, 8, BandShape::BASE, FROM_HASH, W8>(a, cfg);
        default:
            if constexpr (W8) return SS1_ERR_ALGO;  // E4M3 weights need a fixed c
            else return launch_band_cfg<MT, BN, 0, BandShape::BASE, FROM_HASH, false>(a, cfg);
    }
}

template <int MT, bool FROM_HASH, bool W8>
ss1_status launch_band_bn(const ForwardArgs& a, const BandCfg& cfg) {
    switch (a.d.BN) {
        case 32: return launch_band_c<MT, 32, FROM_HASH, W8>(a, cfg);
        case 64: return launch_band_c<MT, 64, FROM_HASH, W8>(a, cfg);
        case 128: return launch_band_c<MT, 128, FROM_HASH, W8>(a, cfg);
        default: return SS1_ERR_ALGO;
    }
}

template <bool FROM_HASH, bool W8>
ss1_status launch_band_t(const ForwardArgs& a) {
    const BandCfg cfg = band_config(a.d, a.M, device_info());
    switch (cfg.MT) {
        case 64: return launch_band_bn<64, FROM_HASH, W8>(a, cfg);
        case 48: return launch_band_bn<48, FROM_HASH, W8>(a, cfg);
        case 32: return launch_band_bn<32, FROM_HASH, W8>(a, cfg);
        default: return SS1_ERR_ALGO;
    }
}

}  // namespace

bool band_supported(const ForwardArgs& a, int min_rows) {
    if (!(a.dtype == SS1_BF16 && a.d.BK % 32 == 0 && (a.d.BN == 32 || a.d.BN == 64 || a.d.BN == 128)))
        return false;
    // E4M3 weights: the forward hash and a fixed c only
    if (a.w_fp8 && !(a.form == PlanForm::Hash && (a.d.c == 1 || a.d.c == 2 || a.d.c == 4 || a.d.c == 8)))
        return false;
    const BandCfg cfg = band_config(a.d, a.M > 0 ? a.M : 1, device_info());
    return cfg.MT >= min_rows;
}

ss1_status launch_band(const ForwardArgs& a) {
    if (a.w_fp8) return a.form == PlanForm::Hash ? launch_band_t<true, true>(a) : SS1_ERR_ALGO;
    return a.form == PlanForm::Hash ? launch_band_t<true, false>(a) : launch_band_t<false, false>(a);
}

bool fused_supported(const ForwardArgs& a) {
    return a.dtype == SS1_BF16 && a.d.BK % 32 == 0 &&
           (a.d.BN == 32 || a.d.BN == 64 || a.d.BN == 128);
}

bool smallm_supported(const ForwardArgs& a) {
    return a.dtype == SS1_BF16 && a.M <= 16 && a.d.BK % 32 == 0 && a.d.BN % 16 == 0;
}

ss1_status launch_generic(const ForwardArgs& a) {
    return a.form == PlanForm::Hash ? launch_generic_t<true>(a) : launch_generic_t<false>(a);
}

ss1_status launch_fused(const ForwardArgs& a) {
    // fp8 weights come with the forward hash only
    if (a.w_fp8) return a.form == PlanForm::Hash ? launch_fused_t<true, true>(a) : SS1_ERR_ALGO;
    return a.form == PlanForm::Hash ? launch_fused_t<false, true>(a) : launch_fused_t<false, false>(a);
}

ss1_status launch_smallm(const ForwardArgs& a) {
    if (a.w_fp8) return a.form == PlanForm::Hash ? launch_smallm_t<true, true>(a) : SS1_ERR_ALGO;
    return a.form == PlanForm::Hash ? launch_smallm_t<false, true>(a) : launch_smallm_t<false, false>(a);
}

ss1_status launch_sketch(const void* x, int32_t x_dtype, const int32_t* plan_i,
                         const int8_t* plan_s, int64_t M, const Dims& d, void* z,
                         int32_t z_dtype, void* stream) {
    const int V = (x_dtype == SS1_BF16) ? 8 : 4;
    const long long items = M * d.Jc * (d.BK / V);
    long long per_group = (items + 255) / 256;
    if (per_group > 4096) per_group = 4096;
    if (per_group < 1) per_group = 1;
    if (d.G > 65535) return SS1_ERR_SHAPE;
    const dim3 grid(static_cast<unsigned>(per_group), static_cast<unsigned>(d.G));
    const size_t lds = plan_lds_bytes(d);
    hipStream_t st = static_cast<hipStream_t>(stream);
    // the sketch kernel reads the forward hash
    if (x_dtype == SS1_BF16 && z_dtype == SS1_BF16)
        hipLaunchKernelGGL((sketch_kernel<uint16_t, true, true>), grid, dim3(256), lds, st,
                           static_cast<const uint16_t*>(x), plan_i, plan_s, z, (int)M, (int)d.K,
                           (int)d.J, (int)d.Jc, d.c, d.BK, (int)d.Kc);
    else if (x_dtype == SS1_BF16)
        hipLaunchKernelGGL((sketch_kernel<uint16_t, false, true>), grid, dim3(256), lds, st,
                           static_cast<const uint16_t*>(x), plan_i, plan_s, z, (int)M, (int)d.K,
                           (int)d.J, (int)d.Jc, d.c, d.BK, (int)d.Kc);
    else
        hipLaunchKernelGGL((sketch_kernel<float, false, true>), grid, dim3(256), lds, st,
                           static_cast<const float*>(x), plan_i, plan_s, z, (int)M, (int)d.K,
                           (int)d.J, (int)d.Jc, d.c, d.BK, (int)d.Kc);
    return launch_status();
}

}  // namespace ss1
