// The SS1 forward with only the compressed contraction on the matrix cores,
// for large M (the SS1 summary page, "Approach": the input is sketched down by
// c with signed chunk additions, then multiplied by the compressed weight,
// which cuts the multiplies by c).
//
// Block: one neuron group (BN neurons, one hash and sign vector) and BM
// tokens.  K runs in stages of 64 compressed columns (BK % 64 == 0, so a stage
// sits inside one compressed chunk t).  Per stage, direct buffer-to-LDS loads
// bring the c source chunks of x that the group's hash sends to t (BM rows x
// 128 bytes each, ascending source order) and the group's W_c columns of the
// stage (BN rows x 128 bytes).  The sketch is formed on the matrix cores: a
// 16x16x32 bf16 MFMA against a signed one-hot selection adds two signed
// sources exactly (sketch_selector in ss1_msketch.h), pairs of sources
// accumulate in float32, and the sum is rounded to bf16 (RNE) as it becomes the
// contraction's operand.  The contraction is y^T = W_c z^T with the weight
// rows placed in a permuted order, so each lane ends with 4*BN/16 consecutive
// neurons of one token and stores them as 16-byte vectors.
//
// Why this shape on gfx950: the vector ALUs run a float32 add at 1/32 of the
// bf16 MFMA rate per element, so a sketch formed on them (widen, signed add,
// round) costs 2.5x the compressed MFMA time at c = 2 and BN = 64; on the
// matrix cores it costs c/4 of the compressed contraction (16*c multiplies per
// sketch element against BN = 64).  What remains is the gather: each group
// reads its BM x K band of x once, so a compute unit moves 2c/BN bytes of x per
// compressed multiply-add through its load path, against 2/256 per dense
// multiply-add for the fold's 256x256 tiles.
//
// LDS: 2 or 3 stages of (c*BM + BN) rows of 128 bytes (c*BM = 256 or 512;
// the launch shapes are listed at group_shape_dims), the next stages loading
// while one is read.  Rows are XOR-swizzled in 16-byte pieces as in the fold
// kernels; lanes of the second source read the other 16-input half of a
// half-step, so that quarter-waves that may share an LDS cycle read different
// pieces.  (The counters still show about a third of the LDS-active cycles as
// bank conflicts; the kernel is bound by its loads, not by the LDS.)
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>

#include "ss1_device.h"
#include "ss1_dma.h"
#include "ss1_group.h"
#include "ss1_internal.h"
#include "ss1_msketch.h"

namespace ss1 {

namespace {

using namespace dev;

constexpr int kGroupRowBytes = 128;  // 64 bf16 per tile row

// Neuron (inside the group) held by LDS row p of the weight tile: MFMA row
// r = 4a + b of neuron block nb = p / 16 holds neuron a*4*NB + nb*4 + b.
template <int NB>
__device__ __forceinline__ int group_neuron(int p) {
    const int nb = p >> 4;
    const int r = p & 15;
    return (r >> 2) * 4 * NB + nb * 4 + (r & 3);
}

template <int C, int BN, int BM, int NW, int NSTG, bool FROM_HASH>
__global__ __launch_bounds__(NW * 64) void group_kernel(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ w,
                                                        const int32_t* __restrict__ pi,
                                                        const int8_t* __restrict__ ps, uint16_t* __restrict__ y,
                                                        int M, int K, int N, int J, int Jc, int BK, int n_mt,
                                                        int tpb, int act) {
    constexpr int RB = kGroupRowBytes;
    constexpr int NB = BN / 16;          // 16-neuron blocks of the group
    constexpr int TB = BM / 16 / NW;     // 16-token blocks per wave
    constexpr int NP = C / 2;            // source pairs per compressed column
    constexpr int SXR = C * BM;          // x rows per stage (source-major)
    constexpr int SX = SXR * RB;         // x bytes per stage
    constexpr int SB = SX + BN * RB;     // stage bytes
    constexpr int XI = SXR / 8 / NW;     // x wave-loads per wave per stage (8 rows each)
    constexpr int WI = BN / 8 / NW;      // weight wave-loads per wave per stage
    constexpr int DPW = XI + WI;
    static_assert(C % 2 == 0 && C >= 2 && C <= 8, "even c");
    static_assert(TB * 16 * NW == BM && XI * 8 * NW == SXR && WI * 8 * NW == BN, "tile split");
    static_assert(NW % 2 == 0, "the swizzle key must repeat between a wave's loads");
    static_assert(BM % 16 == 0 && NB % 2 == 0, "tile sizes");
    static_assert(NSTG == 2 || NSTG == 3, "stage count");
    // the source of every x wave-load is known at compile time when a wave's
    // loads step through whole tiles
    constexpr bool SRC_CT = BM % (NW * 8) == 0;

    extern __shared__ __attribute__((aligned(16))) uint8_t group_smem[];
    uint32_t* s_src = reinterpret_cast<uint32_t*>(group_smem + NSTG * SB);
    int* s_cnt = reinterpret_cast<int*>(s_src + J);

    // A block is one group and tpb consecutive token tiles, which it runs as
    // one pipeline of stages (the plan staged once, no drain between tiles).
    // Each XCD takes a contiguous range of blocks, groups fastest, so the
    // blocks that run together on an XCD read the same token tiles of x.
    const int G = N / BN;
    const int n_chunks = (n_mt + tpb - 1) / tpb;
    const int bid = xcd_tile(blockIdx.x, n_chunks * G);
    const int g = bid % G;
    const int mt0 = (bid / G) * tpb;
    const int ntile = min(tpb, n_mt - mt0);
    stage_plans<FROM_HASH>(pi, ps, g, 1, J, Jc, C, BK, s_src, s_cnt);  // ends with a barrier

    const int Kc = Jc * BK;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nstage = Kc / 64;   // stages per token tile
    const int ntot = ntile * nstage;

    // ---- direct-to-LDS loads: wave-wide load L fills LDS rows [8L, 8L+8);
    // lane l writes 16 bytes at row 8L + l/8, slot l%8, and so reads piece
    // (l%8) ^ key(row) of that row.  This wave does loads wave, wave+NW, ...;
    // the key repeats every 16 rows, so one lane offset serves all of them.
    const i32x4 wr = dma_rsrc(w + static_cast<size_t>(g) * BN * Kc, static_cast<uint32_t>(static_cast<size_t>(BN) * Kc * 2));
    const int lrow = lane >> 3;
    const int piece = (lane & 7) ^ swz_key<RB>(wave * 8 + lrow);
    uint32_t x_voff[XI];
    int x_src[XI];
#pragma unroll
    for (int ii = 0; ii < XI; ++ii) {
        const int row = (wave + NW * ii) * 8 + lrow;  // LDS row in the x region
        x_src[ii] = SRC_CT ? (ii * NW * 8) / BM : __builtin_amdgcn_readfirstlane(((wave + NW * ii) * 8) / BM);
        x_voff[ii] = static_cast<uint32_t>((row - x_src[ii] * BM) * K + piece * 8) * 2u;
    }
    uint32_t w_voff[WI];
#pragma unroll
    for (int ii = 0; ii < WI; ++ii) {
        const int p = (wave + NW * ii) * 8 + lrow;
        w_voff[ii] = static_cast<uint32_t>(group_neuron<NB>(p) * Kc + piece * 8) * 2u;
    }
    const uint32_t lds0 = lds_address(group_smem);
    auto dma = [&](int S, int buf) {
        const int i = S / nstage;  // token tile of the block
        const int s = S - i * nstage;
        const int m0 = (mt0 + i) * BM;
        const i32x4 xr = dma_rsrc(x + static_cast<size_t>(m0) * K,
                                   static_cast<uint32_t>(static_cast<size_t>(min(BM, M - m0)) * K * 2));
        const int k0 = s * 64;
        const int t = k0 / BK;
        const int ub = k0 - t * BK;
        const uint32_t base = lds0 + static_cast<uint32_t>(buf * SB);
        uint32_t ent[C];
#pragma unroll
        for (int r = 0; r < C; ++r) ent[r] = __builtin_amdgcn_readfirstlane(s_src[t * C + r]);
#pragma unroll
        for (int ii = 0; ii < XI; ++ii) {
            uint32_t e;
            if constexpr (SRC_CT) {
                e = ent[(ii * NW * 8) / BM];
            } else {
                e = ent[0];
#pragma unroll
                for (int r = 1; r < C; ++r) e = x_src[ii] == r ? ent[r] : e;
            }
            const bool absent = (e & kAbsent) != 0;
            const int row0 = (wave + NW * ii) * 8;
            lds_dma16(xr, base + row0 * RB, absent ? kDmaAbsent : x_voff[ii],
                      static_cast<uint32_t>((e & kOffMask) + ub) * 2u);
        }
#pragma unroll
        for (int ii = 0; ii < WI; ++ii) {
            const int row0 = (wave + NW * ii) * 8;
            lds_dma16(wr, base + SX + row0 * RB, w_voff[ii], static_cast<uint32_t>(k0) * 2u);
        }
    };

    // ---- operands.  Lane l reads row (block base + l%16); the swizzle key of
    // that row depends on l%16 only.
    const int li = lane & 15;
    const int q = lane >> 4;
    const int key = swz_key<RB>(li);
    const int tok0 = wave * TB * 16;  // this wave's first token of the tile
    uint4 sel_one, sel_neg;
    sketch_selector_base(li, q, sel_one, sel_neg, true);
    const int ohalf = (q & 1) ^ (q >> 1);  // which 16 of a half-step's 32 inputs this lane reads
    // x operand rows of this lane: source 2p + q/2 (pair p), token tok0 + tb*16 + li
    const int xrow = (q >> 1) * BM + tok0 + li;

    f32x4 acc[NB][TB];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < TB; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](int s, int buf) {  // s: stage inside the token tile
        const int t = (s * 64) / BK;
        uint4 sel[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const uint32_t e0 = __builtin_amdgcn_readfirstlane(s_src[t * C + 2 * p]);
            const uint32_t e1 = __builtin_amdgcn_readfirstlane(s_src[t * C + 2 * p + 1]);
            const uint32_t e = q < 2 ? e0 : e1;
            sel[p] = sketch_selector(sel_one, sel_neg, entry_sign_xor(e), entry_sign(e));
        }
        const uint8_t* X = group_smem + buf * SB + xrow * RB;
        const uint8_t* W = group_smem + buf * SB + SX + li * RB;
        // every operand of the stage is requested before the first MFMA
        bf16x8 wop[2][NB];
        uint4 xa[2][TB][NP], xb[2][TB][NP];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int pa = ((4 * h + 2 * ohalf) ^ key) << 4;
            const int pb = ((4 * h + 2 * ohalf + 1) ^ key) << 4;
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    const uint8_t* r = X + (2 * p * BM + tb * 16) * RB;
                    xa[h][tb][p] = *reinterpret_cast<const uint4*>(r + pa);
                    xb[h][tb][p] = *reinterpret_cast<const uint4*>(r + pb);
                }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                wop[h][nb] = *reinterpret_cast<const bf16x8*>(W + nb * 16 * RB + (((4 * h + q) ^ key) << 4));
        }
        // sketches of both 32-wide halves, then the contraction
        f32x4 d0[2][TB], d1[2][TB];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                d0[h][tb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                d1[h][tb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    const uint4 a = xa[h][tb][p], b = xb[h][tb][p];
                    const uint4 x0 = make_uint4(a.x, a.y, b.x, b.y);
                    const uint4 x1 = make_uint4(a.z, a.w, b.z, b.w);
                    d0[h][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, sel[p]), __builtin_bit_cast(bf16x8, x0), d0[h][tb], 0, 0, 0);
                    d1[h][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, sel[p]), __builtin_bit_cast(bf16x8, x1), d1[h][tb], 0, 0, 0);
                }
            }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                uint4 zp;
                zp.x = pack_bf16(d0[h][tb][0], d0[h][tb][1]);
                zp.y = pack_bf16(d0[h][tb][2], d0[h][tb][3]);
                zp.z = pack_bf16(d1[h][tb][0], d1[h][tb][1]);
                zp.w = pack_bf16(d1[h][tb][2], d1[h][tb][3]);
                const bf16x8 zf = __builtin_bit_cast(bf16x8, zp);
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wop[h][nb], zf, acc[nb][tb], 0, 0, 0);
                __builtin_amdgcn_s_setprio(0);
            }
    };
    auto wait_stage = [&](int ahead) {
        if (NSTG == 3 && ahead >= 1) dma_stage_barrier<DPW>();
        else dma_stage_barrier<0>();
    };

    // epilogue of token tile m0: lane holds neurons q*4*NB + nb*4 + i of token
    // m0 + tok0 + tb*16 + li; the accumulators start again from zero
    const int nbase = g * BN + q * 4 * NB;
    auto store_tile = [&](int m0) {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int m = m0 + tok0 + tb * 16 + li;
            if (m < M) {
                uint16_t* yr = y + static_cast<size_t>(m) * N + nbase;
#pragma unroll
                for (int hh = 0; hh < NB / 2; ++hh) {
                    uint4 o;
                    o.x = pack_bf16(apply_act(acc[2 * hh][tb][0], act), apply_act(acc[2 * hh][tb][1], act));
                    o.y = pack_bf16(apply_act(acc[2 * hh][tb][2], act), apply_act(acc[2 * hh][tb][3], act));
                    o.z = pack_bf16(apply_act(acc[2 * hh + 1][tb][0], act), apply_act(acc[2 * hh + 1][tb][1], act));
                    o.w = pack_bf16(apply_act(acc[2 * hh + 1][tb][2], act), apply_act(acc[2 * hh + 1][tb][3], act));
                    *reinterpret_cast<uint4*>(yr + 8 * hh) = o;
                }
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb][tb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };

    // ---- pipeline over the block's ntot stages (tile-major).  Stage S lives
    // in buffer S % NSTG, loaded NSTG-1 stages ahead.  At the top of stage S a
    // barrier finds stage S loaded (all waves) and every wave done with stage
    // S-1, whose buffer the loads of stage S+NSTG-1 then refill.  A tile's
    // output stores go out after its last stage; they count among the vector
    // memory operations the next barrier's wait covers, which only makes that
    // wait longer.
#pragma unroll
    for (int p = 0; p < NSTG - 1; ++p)
        if (p < ntot) dma(p, p);
    auto step = [&](int S, int buf) {
        wait_stage(min(NSTG - 2, ntot - 1 - S));
        if (S + NSTG - 1 < ntot) dma(S + NSTG - 1, (buf + NSTG - 1) % NSTG);
        const int i = S / nstage;
        const int s = S - i * nstage;
        compute(s, buf);
        if (s == nstage - 1) store_tile((mt0 + i) * BM);
    };
    for (int s0 = 0; s0 < ntot; s0 += NSTG) {
#pragma unroll
        for (int b = 0; b < NSTG; ++b)
            if (s0 + b < ntot) step(s0 + b, b);
    }
}

inline size_t group_lds(int C, int BM, int BN, int NSTG, const Dims& d) {
    const size_t stage = static_cast<size_t>(C * BM + BN) * kGroupRowBytes;
    return NSTG * stage + static_cast<size_t>(d.J) * 4 + static_cast<size_t>(d.Jc) * 4;
}

// Token tiles per block: the count that minimises rounds of blocks times tiles
// per block (the launch's length in tile times), the most tiles per block
// among equals (the fewest plan stagings and pipeline fills).
inline int group_tiles_per_block(long long n_mt, long long G) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    long long best_cost = -1;
    int best = 1;
    for (long long nc = 1; nc <= n_mt; ++nc) {
        const long long tpb = (n_mt + nc - 1) / nc;
        const long long chunks = (n_mt + tpb - 1) / tpb;
        const long long cost = (chunks * G + cus - 1) / cus * tpb;
        if (best_cost < 0 || cost < best_cost || (cost == best_cost && tpb > best)) {
            best_cost = cost;
            best = static_cast<int>(tpb);
        }
    }
    return best;
}

template <int C, int BN, int BM, int NW, int NSTG, bool FROM_HASH>
ss1_status launch_group_shape(const ForwardArgs& a) {
    const Dims& d = a.d;
    const long long n_mt = (a.M + BM - 1) / BM;
    const size_t lds = group_lds(C, BM, BN, NSTG, d);
    auto kern = &group_kernel<C, BN, BM, NW, NSTG, FROM_HASH>;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds)) != hipSuccess)
        return SS1_ERR_HIP;
    const int tpb = group_tiles_per_block(n_mt, d.G);
    const long long blocks = (n_mt + tpb - 1) / tpb * d.G;
    hipLaunchKernelGGL((group_kernel<C, BN, BM, NW, NSTG, FROM_HASH>), dim3(static_cast<unsigned>(blocks)),
                       dim3(NW * 64), lds, static_cast<hipStream_t>(a.stream), static_cast<const uint16_t*>(a.x),
                       static_cast<const uint16_t*>(a.w), a.plan_i, a.plan_s, static_cast<uint16_t*>(a.y), (int)a.M,
                       (int)d.K, (int)d.N, (int)d.J, (int)d.Jc, d.BK, (int)n_mt, tpb, a.act);
    return hipGetLastError() == hipSuccess ? SS1_OK : SS1_ERR_HIP;
}

// Launch shapes (tokens per tile BM, waves, stages), the fastest measured on
// Llama-3-8B gate/up and the square 4096 layer: c = 2 and BN = 64: 256 tokens
// on 8 waves, 2 stages (637 us against 662 for 128 tokens, 3 stages, and 752
// on 4 waves); c = 2 and BN = 128: 128 tokens, 8 waves, 3 stages; c = 4: 128
// tokens, 8 waves, 2 stages (178.8 us on the square layer against 228.2 for
// 64 tokens on 4 waves); c = 8: 64 tokens, 4 waves, 2 stages (201.5 against
// 325.7 for 32 tokens on 2 waves).  With BN = 128 at c >= 4 those do not fit
// in LDS, and three stages of 256 rows of x on 4 or 2 waves run instead.
inline void group_shape_dims(int c, int BN, int* BM, int* NSTG) {
    if (c == 2) {
        *BM = BN == 64 ? 256 : 128;
        *NSTG = BN == 64 ? 2 : 3;
    } else {
        *BM = BN == 64 ? 512 / c : 256 / c;
        *NSTG = BN == 64 ? 2 : 3;
    }
}

template <int C, int BN, bool FROM_HASH>
ss1_status launch_group_cfg(const ForwardArgs& a) {
    if constexpr (C == 2) {
        if constexpr (BN == 64) return launch_group_shape<2, 64, 256, 8, 2, FROM_HASH>(a);
        else return launch_group_shape<2, BN, 128, 8, 3, FROM_HASH>(a);
    } else if constexpr (C == 4) {
        if constexpr (BN == 64) return launch_group_shape<4, 64, 128, 8, 2, FROM_HASH>(a);
        else return launch_group_shape<4, BN, 64, 4, 3, FROM_HASH>(a);
    } else {
        if constexpr (BN == 64) return launch_group_shape<8, 64, 64, 4, 2, FROM_HASH>(a);
        else return launch_group_shape<8, BN, 32, 2, 3, FROM_HASH>(a);
    }
}

template <int BN, bool FROM_HASH>
ss1_status launch_group_c(const ForwardArgs& a) {
    switch (a.d.c) {
        case 2: return launch_group_cfg<2, BN, FROM_HASH>(a);
        case 4: return launch_group_cfg<4, BN, FROM_HASH>(a);
        case 8: return launch_group_cfg<8, BN, FROM_HASH>(a);
        default: return SS1_ERR_ALGO;
    }
}

template <bool FROM_HASH>
ss1_status launch_group_t(const ForwardArgs& a) {
    return a.d.BN == 128 ? launch_group_c<128, FROM_HASH>(a) : launch_group_c<64, FROM_HASH>(a);
}

}  // namespace

bool group_supported(const ForwardArgs& a) {
    if (!(a.dtype == SS1_BF16 && !a.w_fp8 && a.d.BK % 64 == 0 && (a.d.BN == 64 || a.d.BN == 128) &&
          (a.d.c == 2 || a.d.c == 4 || a.d.c == 8)))
        return false;
    int dev = 0, lds_max = 64 * 1024;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && v > 0)
            lds_max = v;
    }
    int BM = 0, NSTG = 0;
    group_shape_dims(a.d.c, a.d.BN, &BM, &NSTG);
    if (group_lds(a.d.c, BM, a.d.BN, NSTG, a.d) > static_cast<size_t>(lds_max)) return false;
    const long long blocks = (std::max<int64_t>(a.M, 1) + BM - 1) / BM * a.d.G;
    // byte offsets of x rows inside a tile and of W_c rows inside a group
    return blocks <= 0x7FFFFFFFLL && BM * a.d.K * 2 < (1LL << 31) && a.d.BN * a.d.Kc * 2 < (1LL << 31);
}

ss1_status launch_group(const ForwardArgs& a) {
    return a.form == PlanForm::Hash ? launch_group_t<true>(a) : launch_group_t<false>(a);
}

}  // namespace ss1
