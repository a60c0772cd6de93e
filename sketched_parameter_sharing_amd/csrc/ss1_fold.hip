// The SS1 forward as one dense-shaped contraction: y = x * B^T, where B is the
// layer's expanded weight, B[n][j*BK + u] = sign_g(j) * W_c[n][h_g(j)*BK + u]
// for neuron n of group g (the SS1 summary page, "Approach": the sketch is a
// linear map S_g of x, so W_c * (S_g x) = (W_c S_g) x, and W_c S_g places each
// compressed chunk of W_c, sign-flipped, at every input chunk that hashes to
// it).  B is never written to memory: each k-stage loads the W_c chunk that
// the stage's input chunk maps to straight into the LDS weight tile, and the
// chunk's sign is applied to the bf16 sign bits as the operand leaves LDS.
//
// Why this form on gfx950: the sketch of x costs VALU work (a widen, a signed
// add and a rounding per element, per group) whose throughput on CDNA4 is about
// 1/64 of the MFMA rate, so sketching every group's input costs more than the
// c-fold MFMA work it saves.  Here every multiply runs on the matrix cores
// (K/Kc = c times the compressed work) and no element of x is gathered per
// group; what stays compressed is the weight in HBM (N x Kc) and its traffic.
// The sums also differ from the sketch kernels in rounding only: there the
// sketch is rounded to bf16 before the MFMA, here nothing is rounded before
// the float32 accumulators.
//
// Block: WM x WN waves (8 or 4), output tile BM tokens x BNB neurons (BNB a
// multiple of BN, so a tile holds whole groups).  K runs in stages of KS = 64
// (BK % 64 == 0, so a stage sits inside one input chunk j).  Stages reach LDS
// by direct buffer-to-LDS loads (no registers, no LDS write instructions),
// NSTG buffers deep, loaded NSTG-1 stages ahead.  Each
// 16-byte piece of a tile row sits at a slot XOR-swizzled by the row, which
// keeps the 16 rows read by one quarter-wave on distinct LDS banks.  A stage's
// weight rows are the W_c chunk that its input chunk maps to (the load offset
// carries it; an absent source points past the buffer and loads zeros), and
// the chunk's sign is applied to the weight operand as it leaves LDS.  The
// MFMA computes the transposed tile y^T = B x^T with each wave's weight rows
// placed in a permuted order, so that every lane ends up holding 4*FN
// consecutive neurons of one token and stores them as 16-byte vectors.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>
#include <cmath>

#include "ss1_device.h"
#include "ss1_dma.h"
#include "ss1_internal.h"

namespace ss1 {

namespace {

using namespace dev;

// Neuron (inside a wave's tile of 16*FN) held by LDS row p of that tile:
// MFMA row r = 4a + b of neuron block nb = p / 16 holds neuron a*4*FN + nb*4 + b.
template <int FN>
__device__ __forceinline__ int fold_neuron(int p) {
    const int nb = p >> 4;
    const int r = p & 15;
    return (r >> 2) * 4 * FN + nb * 4 + (r & 3);
}

// Plan of the block's groups in LDS, per (group gl of the tile, input chunk j):
// s_off = byte offset inside a W_c row of the chunk j maps to (t*BK*WB, WB
// bytes per stored weight), or
// kFoldAbsent for an absent source; s_sgn = 0x80008000 for a negative sign,
// else 0.  Hash form: pi/ps are hash/sign [G][J]; index form: idx/isign
// [G][Jc][c].  Entries out of range leave the source absent.
constexpr uint32_t kFoldAbsent = kDmaAbsent;  // plus any in-tile offset: past the extent

template <bool FROM_HASH, int WB>
__device__ void stage_fold_plan(const int32_t* __restrict__ pi, const int8_t* __restrict__ ps, int g0, int ngr,
                                int J, int Jc, int c, int BK, uint32_t* s_off, uint32_t* s_sgn) {
    const int tid = threadIdx.x;
    const int nt = blockDim.x;
    const int total = ngr * J;
    if (FROM_HASH) {
        const int32_t* gi = pi + static_cast<size_t>(g0) * J;
        const int8_t* gs = ps + static_cast<size_t>(g0) * J;
        for (int e = tid; e < total; e += nt) {
            const int t = gi[e];
            const int s = gs[e];
            const bool ok = t >= 0 && t < Jc && (s == 1 || s == -1);
            s_off[e] = ok ? static_cast<uint32_t>(t * BK) * WB : kFoldAbsent;
            s_sgn[e] = (ok && s < 0) ? 0x80008000u : 0u;
        }
    } else {
        for (int e = tid; e < total; e += nt) {
            s_off[e] = kFoldAbsent;
            s_sgn[e] = 0u;
        }
        __syncthreads();
        const int per = Jc * c;
        const int32_t* gi = pi + static_cast<size_t>(g0) * per;
        const int8_t* gs = ps + static_cast<size_t>(g0) * per;
        for (int e = tid; e < ngr * per; e += nt) {
            const int gl = e / per;
            const int t = (e - gl * per) / c;
            const int j = gi[e];
            const int s = gs[e];
            if (j >= 0 && j < J && (s == 1 || s == -1)) {
                s_off[gl * J + j] = static_cast<uint32_t>(t * BK) * WB;
                s_sgn[gl * J + j] = s < 0 ? 0x80008000u : 0u;
            }
        }
    }
    __syncthreads();
}

template <int BM, int BNB, int WM, int WN, int KS, int NSTG, bool W8, bool FROM_HASH>
__global__ __launch_bounds__(WM * WN * 64) void fold_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                   const int32_t* __restrict__ pi, const int8_t* __restrict__ ps,
                                                   uint16_t* __restrict__ y, int M, int K, int N, int J, int Jc,
                                                   int c, int BK, int BN, int n_mt, int act, int n_base,
                                                   int n_cols, const float* __restrict__ wscale) {
    constexpr int NWV = WM * WN;                  // waves per block
    constexpr int TMW = BM / WM, TNW = BNB / WN;  // wave tile: tokens x neurons
    constexpr int FM = TMW / 16, FN = TNW / 16;   // 16x16 MFMA blocks per wave
    static_assert(FM * 16 == TMW && FN * 16 == TNW && FN % 2 == 0, "wave tile");
    constexpr int RB = KS * 2;                    // bytes per x tile row
    constexpr int CPR = RB / 16;                  // 16-byte pieces per row
    constexpr int RPI = 1024 / RB;                // rows filled by one wave-wide load
    // weight tile rows: KS weights of WB bytes (bf16, or E4M3 codes with W8)
    constexpr int WB = W8 ? 1 : 2;
    constexpr int RBW = KS * WB, CPRW = RBW / 16, RPIW = 1024 / RBW;
    constexpr int XI = BM / RPI / NWV;            // x loads per wave per stage
    constexpr int WI = BNB / RPIW / NWV;          // weight loads per wave per stage
    constexpr int DPW = XI + WI;
    static_assert(XI * RPI * NWV == BM && WI * RPIW * NWV == BNB, "tile rows must split over the waves");
    static_assert((NWV * RPI) % 16 == 0 && (NWV * RPIW) % 16 == 0,
                  "the swizzle key must repeat between a wave's loads");
    static_assert(!W8 || KS == 64, "fp8 weights with 64-wide stages");
    static_assert(NSTG >= 2 && NSTG <= 4, "stage count");
    static_assert(KS == 32 || KS == 64, "a stage is one or two 32-wide halves");
    constexpr int HALVES = KS / 32;
    constexpr int SX = BM * RB, SB = SX + BNB * RBW;   // x tile bytes, stage bytes

    extern __shared__ __attribute__((aligned(16))) uint8_t fold_smem[];
    uint32_t* s_off = reinterpret_cast<uint32_t*>(fold_smem + NSTG * SB);

    // Tile order: each XCD takes a contiguous range of tiles (xcd_tile); in
    // that range tiles go in column-major strips of GM row tiles, so the
    // blocks running together on one XCD share a few x row tiles and a few
    // weight column tiles in its L2.
    // (the launch covers neurons [n_base, n_base + n_cols))
    constexpr int GM = 4;
    const int n_nt = n_cols / BNB;
    const int tile = xcd_tile(blockIdx.x, n_mt * n_nt);
    const int strip = tile / (GM * n_nt);
    const int gm = min(GM, n_mt - strip * GM);
    const int rem = tile - strip * GM * n_nt;
    const int mt = strip * GM + rem % gm;
    const int nt = rem / gm;
    const int m0 = mt * BM;
    const int n0 = n_base + nt * BNB;
    const int ngr = BNB / BN;
    uint32_t* s_sgn = s_off + ngr * J;
    const int Kc = Jc * BK;
    stage_fold_plan<FROM_HASH, WB>(pi, ps, n0 / BN, ngr, J, Jc, c, BK, s_off, s_sgn);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int nstage = K / KS;

    // ---- direct-to-LDS loads.  Wave-wide load i of a tile fills rows
    // [i*RPI, i*RPI + RPI); lane l writes 16 bytes at row i*RPI + l/CPR, slot
    // l%CPR, and so reads piece (l%CPR) ^ key(row) of that row.  This wave
    // does loads wave, wave+NWV, ...; the key repeats every 16 rows, so one
    // lane offset serves all of them.
    const i32x4 xr = dma_rsrc(x + static_cast<size_t>(m0) * K,
                               static_cast<uint32_t>(static_cast<size_t>(min(BM, M - m0)) * K * 2));
    const i32x4 wr = dma_rsrc(reinterpret_cast<const uint8_t*>(w) + static_cast<size_t>(n0) * Kc * WB,
                               static_cast<uint32_t>(static_cast<size_t>(BNB) * Kc * WB));
    const int lrow = lane / CPR;
    const int piece = (lane % CPR) ^ swz_key<RB>(wave * RPI + lrow);
    const uint32_t x_voff = static_cast<uint32_t>(lrow * K + piece * 8) * 2u;
    uint32_t w_voff[WI];
    int w_gl[WI];  // group (inside the tile) of this lane's weight row, per load
    const int lroww = lane / CPRW;
    const int piecew = (lane % CPRW) ^ swz_key<RBW>(wave * RPIW + lroww);
#pragma unroll
    for (int ii = 0; ii < WI; ++ii) {
        const int p = (wave + NWV * ii) * RPIW + lroww;               // LDS row in the weight tile
        const int n = (p / TNW) * TNW + fold_neuron<FN>(p % TNW);    // neuron inside the tile
        w_voff[ii] = static_cast<uint32_t>(n * Kc * WB + piecew * 16);
        w_gl[ii] = n / BN;
    }
    const uint32_t lds0 = lds_address(fold_smem);
    auto dma = [&](int s, int buf) {
        const int k0 = s * KS;
        const int j = k0 / BK;
        const uint32_t u0w = static_cast<uint32_t>(k0 - j * BK) * WB;  // bytes into the chunk
        const uint32_t base = lds0 + static_cast<uint32_t>(buf * SB);
        uint32_t off[WI];
#pragma unroll
        for (int ii = 0; ii < WI; ++ii) off[ii] = s_off[w_gl[ii] * J + j];
#pragma unroll
        for (int ii = 0; ii < XI; ++ii) {
            const int row0 = (wave + NWV * ii) * RPI;
            lds_dma16(xr, base + row0 * RB, x_voff + static_cast<uint32_t>(row0 * K * 2),
                      static_cast<uint32_t>(k0 * 2));
        }
#pragma unroll
        for (int ii = 0; ii < WI; ++ii) {
            const int row0 = (wave + NWV * ii) * RPIW;
            lds_dma16(wr, base + SX + row0 * RBW, w_voff[ii] + off[ii] + u0w, 0u);
        }
    };

    // ---- operands.  Lane l reads row (block base + l%16) at logical piece
    // kk/8 + l/16; the key of that row depends on l%16 only.
    const int fr = lane & 15;
    const int q = lane >> 4;
    const int key = swz_key<RB>(fr);
    // group (inside the tile) of the weight rows this lane feeds to the MFMA
    const int sg_gl = (wn * TNW + (fr >> 2) * 4 * FN) / BN;

    f32x4 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // Operands of one 32-wide half of a stage: FN weight blocks (sign applied)
    // and FM token blocks.
    struct Ops {
        bf16x8 w[FN], x[FM];
    };
    // piece of the weight row holding this lane's 8 weights (E4M3: 8 bytes, in
    // half of a 16-byte piece; the key of 64-byte rows depends on l%16 only)
    auto w_off = [&](int half) {
        if constexpr (W8) {
            const int byte = half * 32 + 8 * q;
            return (((byte >> 4) ^ swz_key<RBW>(fr)) << 4) | (byte & 8);
        } else {
            return ((half * 4 + q) ^ key) * 16;
        }
    };
    auto read_ops = [&](int s, int buf, int half, Ops& o) {
        const uint32_t sx = s_sgn[sg_gl * J + (s * KS) / BK];
        const int off = ((half * 4 + q) ^ key) * 16;  // piece half*4 + q of CPR
        const uint8_t* X = fold_smem + buf * SB + (wm * TMW + fr) * RB + off;
        const uint8_t* W = fold_smem + buf * SB + SX + (wn * TNW + fr) * RBW + w_off(half);
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            uint4 v;
            if constexpr (W8) {
                v = fp8x8_to_bf16x8(*reinterpret_cast<const uint2*>(W + i * 16 * RBW));
            } else {
                v = *reinterpret_cast<const uint4*>(W + i * 16 * RBW);
            }
            v.x ^= sx;
            v.y ^= sx;
            v.z ^= sx;
            v.w ^= sx;
            o.w[i] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int jj = 0; jj < FM; ++jj) o.x[jj] = *reinterpret_cast<const bf16x8*>(X + jj * 16 * RB);
    };
    auto mma = [&](const Ops& o) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int jj = 0; jj < FM; ++jj)
                acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.w[i], o.x[jj], acc[i][jj], 0, 0, 0);
    };
    // wait until stage s's loads (all waves) have landed; `ahead` stages were
    // issued after it
    auto wait_stage = [&](int ahead) {
        if (ahead >= 2) dma_stage_barrier<2 * DPW>();
        else if (ahead == 1) dma_stage_barrier<DPW>();
        else dma_stage_barrier<0>();
    };

    // ---- pipeline.  Stage s lives in buffer s % NSTG.
    // Loaded NSTG-1 stages ahead.  At the top of stage s a barrier finds
    // stage s loaded (all waves) and every wave done with stage s-1, whose
    // buffer the loads of stage s+NSTG-1 then refill.
#pragma unroll
    for (int p = 0; p < NSTG - 1; ++p)
        if (p < nstage) dma(p, p);
    auto step = [&](int s, int buf) {
        wait_stage(min(NSTG - 2, nstage - 1 - s));
        if (s + NSTG - 1 < nstage) dma(s + NSTG - 1, (buf + NSTG - 1) % NSTG);
        Ops o[HALVES];
#pragma unroll
        for (int h = 0; h < HALVES; ++h) read_ops(s, buf, h, o[h]);
        // raised issue priority while this wave's MFMAs go out: the other wave
        // on the SIMD, in its LDS reads or barrier, does not split the run
        // (measured 4-5% on the square 4096 layer, neutral on the others)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int h = 0; h < HALVES; ++h) mma(o[h]);
        __builtin_amdgcn_s_setprio(0);
    };
    for (int s0 = 0; s0 < nstage; s0 += NSTG) {
#pragma unroll
        for (int b = 0; b < NSTG; ++b)
            if (s0 + b < nstage) step(s0 + b, b);
    }

    // epilogue: lane holds neurons wn*TNW + (lane/16)*4*FN + nb*4 + i of token
    // wm*TMW + mb*16 + lane%16
    const int nbase = n0 + wn * TNW + q * 4 * FN;
#pragma unroll
    for (int mb = 0; mb < FM; ++mb) {
        const int m = m0 + wm * TMW + mb * 16 + fr;
        if (m >= M) continue;
        uint16_t* yr = y + static_cast<size_t>(m) * N + nbase;
#pragma unroll
        for (int h = 0; h < FN / 2; ++h) {
            float v[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[i] = acc[2 * h][mb][i];
                v[4 + i] = acc[2 * h + 1][mb][i];
            }
            if constexpr (W8) {  // the rows' E4M3 scales
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] *= wscale[nbase + 8 * h + i];
            }
            uint4 o;
            o.x = pack_bf16(apply_act(v[0], act), apply_act(v[1], act));
            o.y = pack_bf16(apply_act(v[2], act), apply_act(v[3], act));
            o.z = pack_bf16(apply_act(v[4], act), apply_act(v[5], act));
            o.w = pack_bf16(apply_act(v[6], act), apply_act(v[7], act));
            *reinterpret_cast<uint4*>(yr + 8 * h) = o;
        }
    }
}

// ============================================================ fp8 fold kernel
// The fold with both operands in OCP E4M3 (x quantized per token row, W_c per
// neuron row, each with a float32 scale) on the gfx950 fp8 matrix cores:
// y[m][n] = xs[m] * ws[n] * sum_k e4m3(xq[m][k]) * B8[n][k], with B8 the
// expanded E4M3 weight (codes of W_c at each input chunk's compressed chunk,
// the chunk's sign on the code's sign bit).  Products of two E4M3 values are
// exact in float32, which accumulates them.
//
// Block: 8 waves (2 x 4), tile 256 tokens x 256 neurons (whole groups), wave
// tile 128 x 64.  K runs in stages of 128 inputs (128 bytes of a token row);
// per stage the MFMA is v_mfma_scale_f32_16x16x128_f8f6f4 (unit scales): each
// lane feeds 32 bytes of one row, at byte 32*(lane/16) of the stage, on both
// operands.  The x tile [256][128 B] comes in 8-row loads (whole 128-byte
// rows); the weight tile comes as two [256][64 B] halves, one per 64 inputs
// (BK % 64 == 0, so a half sits inside one input chunk), each row's half at
// the compressed chunk its group maps that input chunk to; an absent source
// points past the buffer and loads zeros.  The half's sign goes onto the
// weight operand as it leaves LDS (lanes 0-31 read the first half, 32-63 the
// second).  Two LDS stages, the next one loading during the current one.
template <int NSTG>
__global__ __launch_bounds__(512) void fold8_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ xs,
                                                   const uint8_t* __restrict__ wq, const float* __restrict__ ws,
                                                   const int32_t* __restrict__ hash, const int8_t* __restrict__ sign,
                                                   uint16_t* __restrict__ y, int M, int K, int N, int J, int Jc,
                                                   int BK, int BN, int n_mt, int act) {
    constexpr int BM = 256, BNB = 256, WM = 2, WN = 4, NWV = 8;
    constexpr int TMW = BM / WM, TNW = BNB / WN;  // 128 x 64
    constexpr int FM = TMW / 16, FN = TNW / 16;   // 8 x 4
    constexpr int KS = 128;                       // inputs (bytes) per stage
    constexpr int RBX = 128, RPIX = 8;            // x tile: 128-byte rows, 8 rows per wave-wide load
    constexpr int RBW = 64, RPIW = 16;            // weight halves: 64-byte rows, 16 per load
    constexpr int XI = BM / RPIX / NWV;           // 4 x loads per wave per stage
    constexpr int WI = 2 * BNB / RPIW / NWV;      // 4 weight loads per wave per stage
    constexpr int DPW = XI + WI;
    constexpr int SX = BM * RBX;                  // 32 KB
    constexpr int SWH = BNB * RBW;                // 16 KB per weight half
    constexpr int SB = SX + 2 * SWH;              // 64 KB per stage

    extern __shared__ __attribute__((aligned(16))) uint8_t fold_smem[];
    uint32_t* s_off = reinterpret_cast<uint32_t*>(fold_smem + NSTG * SB);

    constexpr int GM = 4;
    const int n_nt = N / BNB;
    const int tile = xcd_tile(blockIdx.x, n_mt * n_nt);
    const int strip = tile / (GM * n_nt);
    const int gm = min(GM, n_mt - strip * GM);
    const int rem = tile - strip * GM * n_nt;
    const int mt = strip * GM + rem % gm;
    const int nt = rem / gm;
    const int m0 = mt * BM;
    const int n0 = nt * BNB;
    const int ngr = BNB / BN;
    uint32_t* s_sgn = s_off + ngr * J;
    const int Kc = Jc * BK;
    stage_fold_plan<true, 1>(hash, sign, n0 / BN, ngr, J, Jc, 1, BK, s_off, s_sgn);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int nstage = K / KS;

    const i32x4 xr = dma_rsrc(xq + static_cast<size_t>(m0) * K,
                              static_cast<uint32_t>(static_cast<size_t>(min(BM, M - m0)) * K));
    const i32x4 wr = dma_rsrc(wq + static_cast<size_t>(n0) * Kc, static_cast<uint32_t>(static_cast<size_t>(BNB) * Kc));
    // x loads: load i = wave + NWV*ii fills rows i*8 .. i*8+7; the key of a
    // row repeats every 16 rows and NWV*8 is a multiple of 16
    const int lrx = lane >> 3;
    const int pcx = (lane & 7) ^ swz_key<RBX>(wave * RPIX + lrx);
    const uint32_t x_voff = static_cast<uint32_t>(lrx * K + pcx * 16);
    // weight loads: load i = wave + NWV*ii < 32; half i / 16, rows (i % 16)*16
    // .. +15 of that half; row p holds neuron (p/64)*64 + fold_neuron(p % 64)
    const int lrw = lane >> 2;
    const int pcw = (lane & 3) ^ swz_key<RBW>(lrw);
    uint32_t w_voff[WI];
    int w_gl[WI];
#pragma unroll
    for (int ii = 0; ii < WI; ++ii) {
        const int i = wave + NWV * ii;
        const int p = (i % 16) * RPIW + lrw;
        const int n = (p / TNW) * TNW + fold_neuron<FN>(p % TNW);
        w_voff[ii] = static_cast<uint32_t>(n * Kc + pcw * 16);
        w_gl[ii] = n / BN;
    }
    const uint32_t lds0 = lds_address(fold_smem);
    auto dma = [&](int s, int buf) {
        const int k0 = s * KS;
        const uint32_t base = lds0 + static_cast<uint32_t>(buf * SB);
#pragma unroll
        for (int ii = 0; ii < XI; ++ii) {
            const int row0 = (wave + NWV * ii) * RPIX;
            lds_dma16(xr, base + row0 * RBX, x_voff + static_cast<uint32_t>(row0 * K), static_cast<uint32_t>(k0));
        }
#pragma unroll
        for (int ii = 0; ii < WI; ++ii) {
            const int i = wave + NWV * ii;
            const int h = i / 16;                      // weight half (compile-time per ii and wave parity)
            const int kh = k0 + 64 * h;                // first input of the half
            const int j = kh / BK;
            const uint32_t off = s_off[w_gl[ii] * J + j];
            lds_dma16(wr, base + SX + h * SWH + (i % 16) * RPIW * RBW,
                      off == kFoldAbsent ? kFoldAbsent : w_voff[ii] + off + static_cast<uint32_t>(kh - j * BK), 0u);
        }
    };

    // operands: lane l (q = l/16) holds row (block base + l%16) at stage
    // inputs 16q .. 16q+15 and 64+16q .. 64+16q+15: x pieces q and q+4 of its
    // 128-byte row, and piece q of its 64-byte row in each weight half.  The
    // MFMA sums over k, so any assignment of the 128 inputs to lanes and
    // registers serves as long as both operands use the same one; this one
    // has the four quarter-waves of each read on consecutive pieces.
    const int fr = lane & 15;
    const int q = lane >> 4;
    const int keyx = swz_key<RBX>(fr);
    const int keyw = swz_key<RBW>(fr);
    const int sg_gl = (wn * TNW + (fr >> 2) * 4 * FN) / BN;

    f32x4 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int jj = 0; jj < FM; ++jj) acc[i][jj] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    typedef int i32x8 __attribute__((ext_vector_type(8)));
    auto step = [&](int s, int buf) {
        if (nstage - 1 - s >= 1 && NSTG >= 3) dma_stage_barrier<DPW>();
        else dma_stage_barrier<0>();
        if (s + NSTG - 1 < nstage) dma(s + NSTG - 1, (buf + NSTG - 1) % NSTG);
        const uint8_t* S = fold_smem + buf * SB;
        // signs of the input chunks of the stage's two 64-input halves
        const uint32_t sx0 = s_sgn[sg_gl * J + (s * KS) / BK] ? 0x80808080u : 0u;
        const uint32_t sx1 = s_sgn[sg_gl * J + (s * KS + 64) / BK] ? 0x80808080u : 0u;
        i32x8 wv[FN];
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const uint8_t* W = S + SX + (wn * TNW + i * 16 + fr) * RBW + ((q ^ keyw) << 4);
            const uint4 a = *reinterpret_cast<const uint4*>(W);
            const uint4 b = *reinterpret_cast<const uint4*>(W + SWH);
            wv[i] = i32x8{static_cast<int>(a.x ^ sx0), static_cast<int>(a.y ^ sx0), static_cast<int>(a.z ^ sx0),
                          static_cast<int>(a.w ^ sx0), static_cast<int>(b.x ^ sx1), static_cast<int>(b.y ^ sx1),
                          static_cast<int>(b.z ^ sx1), static_cast<int>(b.w ^ sx1)};
        }
        // token operands one 16-row block at a time (the next one read while
        // the current block's MFMAs run): 128 accumulators, 32 weight and 16
        // token registers fit the 256 a wave has at two waves per SIMD
        auto xread = [&](int jj) {
            const uint8_t* X = S + (wm * TMW + jj * 16 + fr) * RBX;
            const uint4 a = *reinterpret_cast<const uint4*>(X + ((q ^ keyx) << 4));
            const uint4 b = *reinterpret_cast<const uint4*>(X + (((q + 4) ^ keyx) << 4));
            return i32x8{static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z), static_cast<int>(a.w),
                         static_cast<int>(b.x), static_cast<int>(b.y), static_cast<int>(b.z), static_cast<int>(b.w)};
        };
        i32x8 xv = xread(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int jj = 0; jj < FM; ++jj) {
            const i32x8 xn = jj + 1 < FM ? xread(jj + 1) : xv;
#pragma unroll
            for (int i = 0; i < FN; ++i)
                acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wv[i], xv, acc[i][jj], 0, 0, 0, 127,
                                                                              0, 127);
            xv = xn;
        }
        __builtin_amdgcn_s_setprio(0);
    };
#pragma unroll
    for (int p = 0; p < NSTG - 1; ++p)
        if (p < nstage) dma(p, p);
    for (int s0 = 0; s0 < nstage; s0 += NSTG) {
#pragma unroll
        for (int b = 0; b < NSTG; ++b)
            if (s0 + b < nstage) step(s0 + b, b);
    }

    // epilogue: lane holds neurons wn*64 + (lane/16)*16 + nb*4 + i of token
    // wm*128 + mb*16 + lane%16; y = acc * xs[m] * ws[n]
    const int nbase = n0 + wn * TNW + q * 4 * FN;
    float wsc[4 * FN];
#pragma unroll
    for (int i = 0; i < 4 * FN; ++i) wsc[i] = ws[nbase + i];
#pragma unroll
    for (int mb = 0; mb < FM; ++mb) {
        const int m = m0 + wm * TMW + mb * 16 + fr;
        if (m >= M) continue;
        const float xsm = xs[m];
        uint16_t* yr = y + static_cast<size_t>(m) * N + nbase;
#pragma unroll
        for (int h = 0; h < FN / 2; ++h) {
            float v[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[i] = acc[2 * h][mb][i] * xsm * wsc[8 * h + i];
                v[4 + i] = acc[2 * h + 1][mb][i] * xsm * wsc[8 * h + 4 + i];
            }
            uint4 o;
            o.x = pack_bf16(apply_act(v[0], act), apply_act(v[1], act));
            o.y = pack_bf16(apply_act(v[2], act), apply_act(v[3], act));
            o.z = pack_bf16(apply_act(v[4], act), apply_act(v[5], act));
            o.w = pack_bf16(apply_act(v[6], act), apply_act(v[7], act));
            *reinterpret_cast<uint4*>(yr + 8 * h) = o;
        }
    }
}

// ================================================================ dx kernel
// dx = dy B, with B the expanded weight of the forward (dx[m][j*BK + u] =
// sum_n dy[m][n] sign_g(n)(j) W_c[n][h_g(n)(j)*BK + u]): the same contraction
// with the roles of the two indices swapped.  The kernel computes the
// transposed tile dx^T = B^T dy^T: the weight operand (16 input features x
// 32 neurons) comes out of an LDS tile of W_c rows through ds_read_b64_tr_b16,
// the dy operand (32 neurons x 16 tokens) out of dy rows, so each lane ends
// up with 4 consecutive input features of one token (8-byte stores).
//
// Block: 8 waves (2 x 4), tile BM = 256 or 128 tokens x 256 input features,
// the four 64-feature sub-tiles each inside one input chunk (BK % 64 == 0).
// Reduction over N in stages of 64 neurons, NSTG LDS buffers filled by direct
// loads NSTG-1 stages ahead: the dy tile [256 tokens][64 neurons] and, per sub-tile, the 64
// W_c rows of the stage, each at the chunk its group maps that input chunk to
// (a per (group, sub-tile) table in LDS holds the offset and the sign).  The
// sign goes onto the weight operand as it leaves LDS.

// XOR key (on 16-byte pieces, even values only) of W_c row r in a stage tile:
// with it the 8-byte transposed reads of one 32-lane pass (rows r0..r0+3 and
// r0+8..r0+11, 32 bytes each) land on distinct banks.
__device__ __forceinline__ int dx_tkey(int r) {
    return 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1));
}

template <int BM, int BNB, int WM, int WN, int NSTG>
__device__ __forceinline__ void dxfold_body(int bid, const uint16_t* __restrict__ dy,
                                            const uint16_t* __restrict__ w, const int32_t* __restrict__ hash,
                                            const int8_t* __restrict__ sign, uint16_t* __restrict__ dx, int M,
                                            int K, int N, int J, int Jc, int BK, int BN, int n_mt) {
    constexpr int NWV = WM * WN;
    constexpr int TMW = BM / WM, TNW = BNB / WN;  // wave tile: tokens x input features
    constexpr int FM = TMW / 16, FN = TNW / 16;
    static_assert(TNW == 64, "one 64-feature sub-tile per wave column");
    constexpr int KS = 64, RB = 128, RPI = 8;     // stage of 64 neurons, 128-byte rows
    constexpr int NSUB = BNB / 64;                // 64-feature sub-tiles
    constexpr int XI = BM / RPI / NWV;            // dy loads per wave per stage
    constexpr int WI = NSUB * (KS / RPI) / NWV;   // W_c loads per wave per stage
    constexpr int DPW = XI + WI;
    static_assert(XI * RPI * NWV == BM && WI * NWV == NSUB * (KS / RPI), "loads must split over the waves");
    static_assert((NWV * RPI) % 16 == 0, "the dy swizzle key must repeat between a wave's loads");
    constexpr int SX = BM * RB, SB = SX + NSUB * KS * RB;

    extern __shared__ __attribute__((aligned(16))) uint8_t fold_smem[];
    const int G = N / BN;
    uint32_t* s_off = reinterpret_cast<uint32_t*>(fold_smem + NSTG * SB);
    uint32_t* s_sgn = s_off + G * NSUB;

    constexpr int GM = 4;
    const int n_nt = K / BNB;
    const int tile = xcd_tile(bid, n_mt * n_nt);
    const int strip = tile / (GM * n_nt);
    const int gm = min(GM, n_mt - strip * GM);
    const int rem = tile - strip * GM * n_nt;
    const int mt = strip * GM + rem % gm;
    const int nt = rem / gm;
    const int m0 = mt * BM;
    const int k0 = nt * BNB;
    const int Kc = Jc * BK;

    // table: per group g and sub-tile jj, byte offset of the source columns in
    // a W_c row (or past the buffer for an absent source) and the sign mask
    for (int e = threadIdx.x; e < G * NSUB; e += blockDim.x) {
        const int g = e / NSUB;
        const int kf = k0 + (e - g * NSUB) * 64;
        const int j = kf / BK;
        const int t = hash[static_cast<size_t>(g) * J + j];
        const int sg = sign[static_cast<size_t>(g) * J + j];
        const bool ok = t >= 0 && t < Jc && (sg == 1 || sg == -1);
        s_off[e] = ok ? static_cast<uint32_t>(t * BK + (kf - j * BK)) * 2u : kFoldAbsent;
        s_sgn[e] = (ok && sg < 0) ? 0x80008000u : 0u;
    }
    __syncthreads();

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int nstage = N / KS;

    // dy loads: as the x loads of the forward
    const i32x4 dr = dma_rsrc(dy + static_cast<size_t>(m0) * N,
                               static_cast<uint32_t>(static_cast<size_t>(min(BM, M - m0)) * N * 2));
    const int lrow = lane / 8;
    const int dpiece = (lane % 8) ^ swz_key<RB>(wave * RPI + lrow);
    const uint32_t dy_voff = static_cast<uint32_t>(lrow * N + dpiece * 8) * 2u;
    // W_c loads: load i = wave + NWV*ii fills rows (i % 8)*8 .. +7 of sub-tile i / 8
    const i32x4 wr = dma_rsrc(w, static_cast<uint32_t>(static_cast<size_t>(N) * Kc * 2));
    int w_row[WI], w_sub[WI];
    uint32_t w_base[WI];
#pragma unroll
    for (int ii = 0; ii < WI; ++ii) {
        const int i = wave + NWV * ii;
        w_sub[ii] = i / (KS / RPI);
        w_row[ii] = (i % (KS / RPI)) * RPI + lrow;  // row inside the stage
        const int piece = (lane % 8) ^ dx_tkey(w_row[ii]);
        w_base[ii] = static_cast<uint32_t>(w_row[ii] * Kc + piece * 8) * 2u;
    }
    const uint32_t lds0 = lds_address(fold_smem);
    auto dma = [&](int s, int buf) {
        const int n0 = s * KS;
        const uint32_t base = lds0 + static_cast<uint32_t>(buf * SB);
        uint32_t voff[WI];
#pragma unroll
        for (int ii = 0; ii < WI; ++ii)
            voff[ii] = w_base[ii] + static_cast<uint32_t>(n0) * static_cast<uint32_t>(Kc) * 2u +
                       s_off[((n0 + w_row[ii]) / BN) * NSUB + w_sub[ii]];
#pragma unroll
        for (int ii = 0; ii < XI; ++ii) {
            const int row0 = (wave + NWV * ii) * RPI;
            lds_dma16(dr, base + row0 * RB, dy_voff + static_cast<uint32_t>(row0 * N * 2),
                      static_cast<uint32_t>(n0 * 2));
        }
#pragma unroll
        for (int ii = 0; ii < WI; ++ii) {
            const int i = wave + NWV * ii;
            lds_dma16(wr, base + SX + w_sub[ii] * (KS * RB) + (i % (KS / RPI)) * RPI * RB, voff[ii], 0u);
        }
    };

    const int fr = lane & 15;
    const int q = lane >> 4;
    const int key = swz_key<RB>(fr);

    f32x4 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    struct Ops {
        bf16x8 w[FN], d[FM];
    };
    // transposed weight operand of feature block nb: lane l gets W[rows
    // half*32 + 8q + e][feature nb*16 + l%16]; addressing lane s of a 16-lane
    // group reads row half*32 + 8q + s/4 (+4) at features nb*16 + 4*(s%4)
    const int tr_s = lane & 15;
    auto read_ops = [&](int s, int buf, int half, Ops& o) {
        const int n0 = s * KS;
        const uint32_t sx = s_sgn[((n0 + half * 32 + 8 * q) / BN) * NSUB + wn];
        const uint8_t* D = fold_smem + buf * SB + (wm * TMW + fr) * RB + ((half * 4 + q) ^ key) * 16;
        const uint8_t* W = fold_smem + buf * SB + SX + wn * (KS * RB);
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const int byte = i * 32 + 8 * (tr_s & 3);  // within the 128-byte row
            const int r_lo = half * 32 + 8 * q + (tr_s >> 2);
            const int r_hi = r_lo + 4;
            const uint8_t* plo = W + r_lo * RB + ((((byte >> 4) ^ dx_tkey(r_lo)) << 4) | (byte & 8));
            const uint8_t* phi = W + r_hi * RB + ((((byte >> 4) ^ dx_tkey(r_hi)) << 4) | (byte & 8));
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(plo));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(phi));
            uint4 v;
            v.x = (static_cast<uint32_t>(static_cast<uint16_t>(lo[0])) | (static_cast<uint32_t>(static_cast<uint16_t>(lo[1])) << 16)) ^ sx;
            v.y = (static_cast<uint32_t>(static_cast<uint16_t>(lo[2])) | (static_cast<uint32_t>(static_cast<uint16_t>(lo[3])) << 16)) ^ sx;
            v.z = (static_cast<uint32_t>(static_cast<uint16_t>(hi[0])) | (static_cast<uint32_t>(static_cast<uint16_t>(hi[1])) << 16)) ^ sx;
            v.w = (static_cast<uint32_t>(static_cast<uint16_t>(hi[2])) | (static_cast<uint32_t>(static_cast<uint16_t>(hi[3])) << 16)) ^ sx;
            o.w[i] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int jj = 0; jj < FM; ++jj) o.d[jj] = *reinterpret_cast<const bf16x8*>(D + jj * 16 * RB);
    };
    auto mma = [&](const Ops& o) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int jj = 0; jj < FM; ++jj)
                acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.w[i], o.d[jj], acc[i][jj], 0, 0, 0);
    };
    auto wait_stage = [&](int ahead) {
        if (ahead >= 2) dma_stage_barrier<2 * DPW>();
        else if (ahead == 1) dma_stage_barrier<DPW>();
        else dma_stage_barrier<0>();
    };

#pragma unroll
    for (int p = 0; p < NSTG - 1; ++p)
        if (p < nstage) dma(p, p);
    auto step = [&](int s, int buf) {
        wait_stage(min(NSTG - 2, nstage - 1 - s));
        if (s + NSTG - 1 < nstage) dma(s + NSTG - 1, (buf + NSTG - 1) % NSTG);
        Ops o0, o1;
        read_ops(s, buf, 0, o0);
        read_ops(s, buf, 1, o1);
        __builtin_amdgcn_s_setprio(1);  // as in the forward: keep the MFMA run together
        mma(o0);
        mma(o1);
        __builtin_amdgcn_s_setprio(0);
    };
    for (int s0 = 0; s0 < nstage; s0 += NSTG) {
#pragma unroll
        for (int b = 0; b < NSTG; ++b)
            if (s0 + b < nstage) step(s0 + b, b);
    }

    // epilogue: lane holds features wn*64 + nb*16 + 4q + i of token
    // wm*TMW + mb*16 + lane%16
#pragma unroll
    for (int mb = 0; mb < FM; ++mb) {
        const int m = m0 + wm * TMW + mb * 16 + fr;
        if (m >= M) continue;
        uint16_t* dr_ = dx + static_cast<size_t>(m) * K + k0 + wn * TNW + 4 * q;
#pragma unroll
        for (int nb = 0; nb < FN; ++nb) {
            uint2 o;
            o.x = pack_bf16(acc[nb][mb][0], acc[nb][mb][1]);
            o.y = pack_bf16(acc[nb][mb][2], acc[nb][mb][3]);
            *reinterpret_cast<uint2*>(dr_ + nb * 16) = o;
        }
    }
}

// =============================================================== dW kernel
// dW_c[n][t*BK + u] = sum_m dy[m][n] z_g[m][t*BK + u] with z_g the sketch of x
// = sum over tokens m and the c sources j_r of chunk t of
//   sign_g(j_r) x[m][j_r*BK + u] dy[m][n]:
// a contraction over (m, r) with no sketch formed (the fold of the forward,
// applied on the reduction side).  The kernel computes the transposed tile
// dW_c^T[kc][n] = sum x-chunk^T dy; both operands come out of row-major
// [token][...] LDS tiles through ds_read_b64_tr_b16, and each lane ends with
// 4 consecutive compressed columns of one neuron (8-byte stores).
//
// Block: 8 waves, tile KT compressed columns x 64 neurons inside one group.
// Waves 0-3 and 4-7 cover the tile the same way (4 x 64 columns x 64 neurons
// for KT = 256, 2 x 2 of 64 x 32 for KT = 128) and split each 64-token stage
// into its two 32-token halves; their partial sums meet in LDS at the end.
// Per stage, direct loads bring the dy tile [64 tokens][64 neurons] and, per
// 64-column sub-tile st and source r, the x tile [64 tokens][64 columns] at
// source chunk j_r of that sub-tile's compressed chunk (a table in LDS from
// the block's group plan; a missing source points past x and loads zeros).
// The source's sign goes onto the x operand as it leaves LDS.
template <int KT, int CS, int NSTG>
__device__ __forceinline__ void dwfold_body(int bid, const uint16_t* __restrict__ x, const uint16_t* __restrict__ dy,
                                            const int32_t* __restrict__ hash, const int8_t* __restrict__ sign,
                                            uint16_t* __restrict__ dw, int M, int K, int N, int J, int Jc, int BK,
                                            int BN) {
    constexpr int NWV = 8;
    constexpr int NSUB = KT / 64;                 // 64-column sub-tiles
    constexpr int WM = NSUB, WN = 4 / WM;         // waves of a half: along columns x neurons
    static_assert(WM * WN == 4, "four waves per half");
    constexpr int TNW = 64 / WN;                  // neurons per wave
    constexpr int FA = 4, FB = TNW / 16;          // 16-blocks: columns (64 per wave) x neurons
    constexpr int KS = 64, RB = 128, RPI = 8;     // stage of 64 tokens, 128-byte tile rows
    constexpr int NT = NSUB * CS + 1;             // tiles per stage: x sub-tiles, then dy
    constexpr int LOADS = NT * (KS / RPI);        // wave-wide loads per stage
    static_assert(LOADS % NWV == 0, "loads must split over the waves");
    constexpr int DPW = LOADS / NWV;
    constexpr int TB = KS * RB;                   // bytes per tile
    constexpr int SB = NT * TB;                   // bytes per stage

    extern __shared__ __attribute__((aligned(16))) uint8_t fold_smem[];
    uint32_t* s_xoff = reinterpret_cast<uint32_t*>(fold_smem + NSTG * SB);  // [NSUB][CS]
    uint32_t* s_xsg = s_xoff + NSUB * CS;
    int* s_cnt = reinterpret_cast<int*>(s_xsg + NSUB * CS);
    int* s_j = s_cnt + NSUB;                                                // [NSUB][CS]

    const int Kc = Jc * BK;
    const int n_ct = Kc / KT;
    const int nt = bid / n_ct;                    // 64-neuron tile
    const int kc0 = (bid - nt * n_ct) * KT;
    const int n0 = nt * 64;
    const int g = n0 / BN;

    // sources of each sub-tile's compressed chunk, ascending in j
    const int tid = threadIdx.x;
    for (int e = tid; e < NSUB * CS; e += blockDim.x) s_j[e] = -1;
    for (int e = tid; e < NSUB; e += blockDim.x) s_cnt[e] = 0;
    __syncthreads();
    for (int j = tid; j < J; j += blockDim.x) {
        const int t = hash[static_cast<size_t>(g) * J + j];
        const int sg = sign[static_cast<size_t>(g) * J + j];
        if (t < 0 || t >= Jc || (sg != 1 && sg != -1)) continue;
#pragma unroll
        for (int st = 0; st < NSUB; ++st) {
            if ((kc0 + 64 * st) / BK != t) continue;
            const int slot = atomicAdd(&s_cnt[st], 1);
            if (slot < CS) s_j[st * CS + slot] = sg < 0 ? -(j + 2) : j;  // sign folded into the code
        }
    }
    __syncthreads();
    if (tid < NSUB) {
        int* p = s_j + tid * CS;
        for (int a = 1; a < CS; ++a) {  // insertion sort by chunk; missing sources (-1) go last
            const int v = p[a];
            const int kv = v == -1 ? 0x7FFFFFFF : (v < 0 ? -v - 2 : v);
            int b = a - 1;
            while (b >= 0) {
                const int kb = p[b] == -1 ? 0x7FFFFFFF : (p[b] < 0 ? -p[b] - 2 : p[b]);
                if (kb <= kv) break;
                p[b + 1] = p[b];
                --b;
            }
            p[b + 1] = v;
        }
    }
    __syncthreads();
    for (int e = tid; e < NSUB * CS; e += blockDim.x) {
        const int v = s_j[e];
        const int st = e / CS;
        const int u0 = (kc0 + 64 * st) % BK;
        if (v == -1) {
            s_xoff[e] = kFoldAbsent;
            s_xsg[e] = 0u;
        } else {
            const int j = v < 0 ? -v - 2 : v;
            s_xoff[e] = static_cast<uint32_t>(j * BK + u0) * 2u;
            s_xsg[e] = v < 0 ? 0x80008000u : 0u;
        }
    }
    __syncthreads();

    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = wave / 4;                    // which 32 tokens of a stage
    const int wl = wave % 4;
    const int wm = wl / WN, wn = wl % WN;
    const int nstage = (M + KS - 1) / KS;

    // Loads: load i = wave + NWV*ii fills rows (i % 8)*8 .. +7 of tile i / 8
    // (tiles 0 .. NSUB*CS-1: x sub-tile st = tile / CS, source r = tile % CS;
    // tile NSUB*CS: dy).  Tokens past M lie past both buffers and load zeros.
    const i32x4 xr = dma_rsrc(x, static_cast<uint32_t>(static_cast<size_t>(M) * K * 2));
    const i32x4 dr = dma_rsrc(dy, static_cast<uint32_t>(static_cast<size_t>(M) * N * 2));
    const int lrow = lane / 8;
    int l_tile[DPW];
    uint32_t l_voff[DPW];
#pragma unroll
    for (int ii = 0; ii < DPW; ++ii) {
        const int i = wave + NWV * ii;
        const int row = (i % (KS / RPI)) * RPI + lrow;
        const int piece = (lane % 8) ^ dx_tkey(row);
        l_tile[ii] = i / (KS / RPI);
        l_voff[ii] = l_tile[ii] < NSUB * CS ? static_cast<uint32_t>(row * K + piece * 8) * 2u
                                            : static_cast<uint32_t>(row * N + n0 + piece * 8) * 2u;
    }
    const uint32_t lds0 = lds_address(fold_smem);
    auto dma = [&](int s, int buf) {
        const int m0 = s * KS;
        const uint32_t base = lds0 + static_cast<uint32_t>(buf * SB);
#pragma unroll
        for (int ii = 0; ii < DPW; ++ii) {
            const int i = wave + NWV * ii;
            const uint32_t dst = base + static_cast<uint32_t>(l_tile[ii] * TB + (i % (KS / RPI)) * RPI * RB);
            if (l_tile[ii] < NSUB * CS) {
                // an absent source keeps its offset past the extent (no wrap)
                const uint32_t xo = s_xoff[l_tile[ii]];
                lds_dma16(xr, dst,
                          xo == kFoldAbsent ? kFoldAbsent : l_voff[ii] + xo + static_cast<uint32_t>(m0) * K * 2u, 0u);
            } else {
                lds_dma16(dr, dst, l_voff[ii] + static_cast<uint32_t>(m0) * N * 2u, 0u);
            }
        }
    };

    const int q = lane >> 4;
    const int tr_s = lane & 15;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    // transposed operand of a 16-wide block at byte `col` of a tile's rows:
    // lane l gets rows 32*half + 8q + e (e = 0..7) of column (col/2 + l%16)
    auto read_tr = [&](const uint8_t* T, int col, uint32_t sx) {
        const int byte = col + 8 * (tr_s & 3);
        const int r_lo = half * 32 + 8 * q + (tr_s >> 2);
        const int r_hi = r_lo + 4;
        const uint8_t* plo = T + r_lo * RB + ((((byte >> 4) ^ dx_tkey(r_lo)) << 4) | (byte & 8));
        const uint8_t* phi = T + r_hi * RB + ((((byte >> 4) ^ dx_tkey(r_hi)) << 4) | (byte & 8));
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(plo));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(phi));
        uint4 v;
        v.x = (static_cast<uint32_t>(static_cast<uint16_t>(lo[0])) | (static_cast<uint32_t>(static_cast<uint16_t>(lo[1])) << 16)) ^ sx;
        v.y = (static_cast<uint32_t>(static_cast<uint16_t>(lo[2])) | (static_cast<uint32_t>(static_cast<uint16_t>(lo[3])) << 16)) ^ sx;
        v.z = (static_cast<uint32_t>(static_cast<uint16_t>(hi[0])) | (static_cast<uint32_t>(static_cast<uint16_t>(hi[1])) << 16)) ^ sx;
        v.w = (static_cast<uint32_t>(static_cast<uint16_t>(hi[2])) | (static_cast<uint32_t>(static_cast<uint16_t>(hi[3])) << 16)) ^ sx;
        return __builtin_bit_cast(bf16x8, v);
    };

    f32x4 acc[FA][FB];
#pragma unroll
    for (int i = 0; i < FA; ++i)
#pragma unroll
        for (int j = 0; j < FB; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](int buf) {
        const uint8_t* S = fold_smem + buf * SB;
        bf16x8 bo[FB];
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) bo[fb] = read_tr(S + NSUB * CS * TB, (wn * TNW + fb * 16) * 2, 0u);
#pragma unroll
        for (int r = 0; r < CS; ++r) {
            const int tile = wm * CS + r;
            const uint32_t sx = s_xsg[tile];
            bf16x8 ao[FA];
#pragma unroll
            for (int fa = 0; fa < FA; ++fa) ao[fa] = read_tr(S + tile * TB, fa * 32, sx);
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int fa = 0; fa < FA; ++fa)
#pragma unroll
                for (int fb = 0; fb < FB; ++fb)
                    acc[fa][fb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao[fa], bo[fb], acc[fa][fb], 0, 0, 0);
            __builtin_amdgcn_s_setprio(0);
        }
    };
    auto wait_stage = [&](int ahead) {
        if (ahead >= 2) dma_stage_barrier<2 * DPW>();
        else if (ahead == 1) dma_stage_barrier<DPW>();
        else dma_stage_barrier<0>();
    };

#pragma unroll
    for (int p = 0; p < NSTG - 1; ++p)
        if (p < nstage) dma(p, p);
    auto step = [&](int s, int buf) {
        wait_stage(min(NSTG - 2, nstage - 1 - s));
        if (s + NSTG - 1 < nstage) dma(s + NSTG - 1, (buf + NSTG - 1) % NSTG);
        compute(buf);
    };
    for (int s0 = 0; s0 < nstage; s0 += NSTG) {
#pragma unroll
        for (int b = 0; b < NSTG; ++b)
            if (s0 + b < nstage) step(s0 + b, b);
    }

    // the two halves' partial tiles meet in LDS (the stage buffers are free
    // once every wave has passed this barrier)
    dma_stage_barrier<0>();
    float* red = reinterpret_cast<float*>(fold_smem);
    if (half == 1) {
#pragma unroll
        for (int fa = 0; fa < FA; ++fa)
#pragma unroll
            for (int fb = 0; fb < FB; ++fb)
#pragma unroll
                for (int i = 0; i < 4; ++i) red[((wl * FA + fa) * FB + fb) * 256 + i * 64 + lane] = acc[fa][fb][i];
    }
    __syncthreads();
    if (half == 0) {
        // lane holds columns wm*64 + fa*16 + 4q + i of neuron wn*TNW + fb*16 + lane%16
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) {
            const int n = n0 + wn * TNW + fb * 16 + tr_s;
            uint16_t* dr_ = dw + static_cast<size_t>(n) * Kc + kc0 + wm * 64 + 4 * q;
#pragma unroll
            for (int fa = 0; fa < FA; ++fa) {
                float v[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = acc[fa][fb][i] + red[((wl * FA + fa) * FB + fb) * 256 + i * 64 + lane];
                uint2 o;
                o.x = pack_bf16(v[0], v[1]);
                o.y = pack_bf16(v[2], v[3]);
                *reinterpret_cast<uint2*>(dr_ + fa * 16) = o;
            }
        }
    }
}

template <int BM, int BNB, int WM, int WN, int NSTG>
__global__ __launch_bounds__(WM * WN * 64) void dxfold_kernel(const uint16_t* __restrict__ dy,
                                                              const uint16_t* __restrict__ w,
                                                              const int32_t* __restrict__ hash,
                                                              const int8_t* __restrict__ sign,
                                                              uint16_t* __restrict__ dx, int M, int K, int N, int J,
                                                              int Jc, int BK, int BN, int n_mt) {
    dxfold_body<BM, BNB, WM, WN, NSTG>(blockIdx.x, dy, w, hash, sign, dx, M, K, N, J, Jc, BK, BN, n_mt);
}

template <int KT, int CS, int NSTG>
__global__ __launch_bounds__(512) void dwfold_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ dy,
                                                     const int32_t* __restrict__ hash,
                                                     const int8_t* __restrict__ sign, uint16_t* __restrict__ dw,
                                                     int M, int K, int N, int J, int Jc, int BK, int BN) {
    dwfold_body<KT, CS, NSTG>(blockIdx.x, x, dy, hash, sign, dw, M, K, N, J, Jc, BK, BN);
}

// Both gradients in one launch: blocks [0, n_dw) are dW_c tiles, the rest dx
// tiles.  The two are independent; sharing the grid lets dx tiles fill the
// compute units that a layer's few dW_c tiles leave idle (GPT-2 S: 144 dW_c
// tiles for 256 compute units), and the longer dW_c tiles are dispatched first.
template <int DXBM, int DXNSTG, int KT, int CS, int DWNSTG>
__global__ __launch_bounds__(512) void bwdfold_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                      const int32_t* __restrict__ hash,
                                                      const int8_t* __restrict__ sign,
                                                      const uint16_t* __restrict__ dy, uint16_t* __restrict__ dx,
                                                      uint16_t* __restrict__ dw, int M, int K, int N, int J, int Jc,
                                                      int BK, int BN, int n_mt, int n_dw) {
    if (static_cast<int>(blockIdx.x) < n_dw)
        dwfold_body<KT, CS, DWNSTG>(blockIdx.x, x, dy, hash, sign, dw, M, K, N, J, Jc, BK, BN);
    else
        dxfold_body<DXBM, 256, 2, 4, DXNSTG>(blockIdx.x - n_dw, dy, w, hash, sign, dx, M, K, N, J, Jc, BK, BN,
                                             n_mt);
}

struct FoldCfg {
    int BM, BNB, KS, NSTG;
    size_t lds;
};

// LDS of a fold launch: NSTG stages of the x tile (BM rows of KS bf16) and the
// weight tile (BNB rows of KS weights of WB bytes), plus the plan table.
inline size_t fold_lds(int BM, int BNB, int KS, int NSTG, int WB, const Dims& d) {
    return static_cast<size_t>(NSTG) * (static_cast<size_t>(BM) * KS * 2 + static_cast<size_t>(BNB) * KS * WB) +
           static_cast<size_t>(2) * (BNB / d.BN) * d.J * 4;
}

int device_attribute(hipDeviceAttribute_t attr, int fallback) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fallback;
    if (hipDeviceGetAttribute(&v, attr, dev) != hipSuccess || v <= 0) return fallback;
    return v;
}

int max_lds_per_block() { return device_attribute(hipDeviceAttributeMaxSharedMemoryPerBlock, 64 * 1024); }

// Tile choice (tokens x neurons), the neuron tile a whole number of groups
// that divides N:
//   256 x 256, 8 waves of 128 x 64, 2 stages (two waves per SIMD: one
//              multiplies while the other waits on LDS or a barrier; 3 stages
//              with E4M3 weights, whose weight tile is half the size);
//   256 x 128, 4 waves of 128 x 64, 3 stages, when N is not a multiple of 256;
//   128 x 128, 4 waves of 64 x 64, 4 stages, for M <= 128 or when only 128
//              divides N and M is small.
// 32-wide stages (twice the buffers) when BK % 64 != 0, bf16 weights only.
// Buffer offsets are 32-bit: a tile's rows must span less than 2 GiB.
// (fold_config below may then trade the 256 x 256 tiles for 192 x 256 ones.)
inline FoldCfg fold_config_base(const ForwardArgs& a) {
    const Dims& d = a.d;
    const int WB = a.w_fp8 ? 1 : 2;
    if (d.BK % 32 != 0 || (a.w_fp8 && d.BK % 64 != 0)) return FoldCfg{0, 0, 0, 0, 0};
    auto fits = [&](int BNB) { return BNB % d.BN == 0 && d.N % BNB == 0; };
    int BM = 0, BNB = 0, NSTG = 0, KS = 64;
    if (fits(256) && a.M > 128) {
        BM = 256;
        BNB = 256;
        NSTG = a.w_fp8 ? 3 : 2;
    } else if (fits(128) && a.M > 128) {
        BM = 256;
        BNB = 128;
        NSTG = 3;
    } else if (fits(128)) {
        BM = 128;
        BNB = 128;
        NSTG = 4;
    }
    if (d.BK % KS != 0) {  // 32-wide stages, twice as many buffers
        KS = 32;
        NSTG = std::min(2 * NSTG, 4);
    }
    if (BM == 0) return FoldCfg{0, 0, 0, 0, 0};
    if (static_cast<double>(std::max(BM * d.K * 2, BNB * d.Kc * WB)) >= 2147483648.0) return FoldCfg{0, 0, 0, 0, 0};
    const size_t lds = fold_lds(BM, BNB, KS, NSTG, WB, d);
    if (lds > static_cast<size_t>(max_lds_per_block())) return FoldCfg{0, 0, 0, 0, 0};
    return FoldCfg{BM, BNB, KS, NSTG, lds};
}

template <int BM, int BNB, int WM, int WN, int KS, int NSTG, bool W8, bool FROM_HASH>
ss1_status launch_fold_cfg(const ForwardArgs& a, size_t lds, int64_t n_base, int64_t n_cols) {
    const Dims& d = a.d;
    const int n_mt = static_cast<int>((a.M + BM - 1) / BM);
    const long long blocks = static_cast<long long>(n_mt) * (n_cols / BNB);
    if (blocks > 0x7FFFFFFFLL) return SS1_ERR_SHAPE;
    if (blocks == 0) return SS1_OK;
    auto kern = &fold_kernel<BM, BNB, WM, WN, KS, NSTG, W8, FROM_HASH>;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds)) != hipSuccess)
        return SS1_ERR_HIP;
    hipLaunchKernelGGL((fold_kernel<BM, BNB, WM, WN, KS, NSTG, W8, FROM_HASH>), dim3(static_cast<unsigned>(blocks)),
                       dim3(WM * WN * 64), lds, static_cast<hipStream_t>(a.stream), static_cast<const uint16_t*>(a.x),
                       static_cast<const uint16_t*>(a.w), a.plan_i, a.plan_s, static_cast<uint16_t*>(a.y),
                       (int)a.M, (int)d.K, (int)d.N, (int)d.J, (int)d.Jc, d.c, d.BK, d.BN, n_mt, a.act, (int)n_base,
                       (int)n_cols, a.wscale);
    return hipGetLastError() == hipSuccess ? SS1_OK : SS1_ERR_HIP;
}

// Stages of the 128 x 256 tiles of a split launch's second part.
inline int fold_rest_nstg(const ForwardArgs& a) { return a.w_fp8 ? 4 : 3; }

// A 256 x 256 launch whose tiles end in a partial round splits its neurons: the
// columns [0, main) in 256 x 256 tiles that fill whole rounds of compute units,
// the rest in 128 x 256 tiles (8 waves of 64 x 64) in a second launch, whose
// one round of half-size tiles takes about 0.55 of a full round.  Returns the
// number of neurons of the first launch (N when there is no split).
int64_t fold_main_cols(const ForwardArgs& a, const FoldCfg& cfg) {
    const Dims& d = a.d;
    if (!(cfg.BM == 256 && cfg.BNB == 256 && cfg.KS == 64)) return d.N;
    if (fold_lds(128, 256, 64, fold_rest_nstg(a), a.w_fp8 ? 1 : 2, d) > static_cast<size_t>(max_lds_per_block()))
        return d.N;
    const long long cus = device_attribute(hipDeviceAttributeMultiprocessorCount, 256);
    const long long n_mt = (a.M + 255) / 256, n_nt = d.N / 256;
    const long long tiles = n_mt * n_nt;
    const long long full = tiles / cus;
    if (full == 0 || tiles % cus == 0) return d.N;
    const long long n_main = full * cus / n_mt;
    if (n_main <= 0 || n_main >= n_nt) return d.N;
    auto rounds = [&](long long t) { return static_cast<double>((t + cus - 1) / cus); };
    const double single = rounds(tiles);
    const double split = rounds(n_mt * n_main) + 0.55 * rounds(((a.M + 127) / 128) * (n_nt - n_main));
    return split < 0.97 * single ? n_main * 256 : d.N;
}

// The tile the fold launch uses: fold_config_base's, except that 256 x 256
// tiles become 192 x 256 where that costs less counted in rounds of tiles
// times tile rows (the 256-row launch with its split, where one applies).  The
// 192-row tile runs the same 8 waves on 96 x 64 wave tiles.  GPT-2 L down
// (M = 8192, N = 1280) is the case: 160 tiles of 256 rows leave 96 of 256
// compute units idle for the whole launch; 215 tiles of 192 rows fill one
// round at three quarters of the work per tile.
FoldCfg fold_config(const ForwardArgs& a) {
    const FoldCfg base = fold_config_base(a);
    if (!(base.BM == 256 && base.BNB == 256 && base.KS == 64)) return base;
    const Dims& d = a.d;
    const double cus = device_attribute(hipDeviceAttributeMultiprocessorCount, 256);
    const double M = static_cast<double>(a.M);
    auto rounds = [&](double tiles) { return std::ceil(tiles / cus); };
    const int64_t main = fold_main_cols(a, base);
    const double cost256 =
        256.0 * (main != d.N ? rounds(std::ceil(M / 256) * static_cast<double>(main / 256)) +
                                   0.55 * rounds(std::ceil(M / 128) * static_cast<double>((d.N - main) / 256))
                             : rounds(std::ceil(M / 256) * static_cast<double>(d.N / 256)));
    const double cost192 = 192.0 * rounds(std::ceil(M / 192) * static_cast<double>(d.N / 256));
    if (!(cost192 < cost256)) return base;
    const size_t lds = fold_lds(192, 256, 64, base.NSTG, a.w_fp8 ? 1 : 2, d);
    if (lds > static_cast<size_t>(max_lds_per_block())) return base;
    return FoldCfg{192, 256, 64, base.NSTG, lds};
}

template <bool FROM_HASH, bool W8>
ss1_status launch_fold_t(const ForwardArgs& a) {
    const FoldCfg cfg = fold_config(a);
    const int64_t N = a.d.N;
    constexpr int WB = W8 ? 1 : 2;
    constexpr int NB = W8 ? 3 : 2;       // stages of the 256 x 256 tile
    constexpr int NR = W8 ? 4 : 3;       // stages of the 128 x 256 tile
    if (cfg.BM == 192 && cfg.BNB == 256 && cfg.KS == 64 && cfg.NSTG == NB)
        return launch_fold_cfg<192, 256, 2, 4, 64, NB, W8, FROM_HASH>(a, cfg.lds, 0, N);
    if (cfg.BM == 256 && cfg.BNB == 256) {
        if (cfg.KS == 64 && cfg.NSTG == NB) {
            const int64_t main = fold_main_cols(a, cfg);
            ss1_status st = launch_fold_cfg<256, 256, 2, 4, 64, NB, W8, FROM_HASH>(a, cfg.lds, 0, main);
            if (st != SS1_OK || main == N) return st;
            return launch_fold_cfg<128, 256, 2, 4, 64, NR, W8, FROM_HASH>(a, fold_lds(128, 256, 64, NR, WB, a.d),
                                                                         main, N - main);
        }
        if constexpr (!W8) {
            if (cfg.KS == 32 && cfg.NSTG == 4)
                return launch_fold_cfg<256, 256, 2, 4, 32, 4, W8, FROM_HASH>(a, cfg.lds, 0, N);
        }
    }
    if (cfg.BM == 256 && cfg.BNB == 128) {
        if (cfg.KS == 64) return launch_fold_cfg<256, 128, 2, 2, 64, 3, W8, FROM_HASH>(a, cfg.lds, 0, N);
        if constexpr (!W8) return launch_fold_cfg<256, 128, 2, 2, 32, 4, W8, FROM_HASH>(a, cfg.lds, 0, N);
    }
    if (cfg.BM == 128 && cfg.BNB == 128) {
        if (cfg.KS == 64) return launch_fold_cfg<128, 128, 2, 2, 64, 4, W8, FROM_HASH>(a, cfg.lds, 0, N);
        if constexpr (!W8) return launch_fold_cfg<128, 128, 2, 2, 32, 4, W8, FROM_HASH>(a, cfg.lds, 0, N);
    }
    return SS1_ERR_ALGO;
}

// dx kernel: tiles of BM = 256 tokens (two LDS stages) or 128 (three stages,
// when 256-token tiles would leave most compute units idle) x 256 input
// features; N a multiple of the 64-neuron stage, K of 256, BK of 64, and the
// plan table plus the stages in LDS; 32-bit buffer offsets need the dy rows of
// a tile and W_c under 2 GiB.
int dxfold_bm(int64_t M, const Dims& d) {
    const double cus = device_attribute(hipDeviceAttributeMultiprocessorCount, 256);
    auto eff = [&](int bm) {
        const double tiles = std::ceil(static_cast<double>(M) / bm) * static_cast<double>(d.K / 256);
        return tiles / (std::ceil(tiles / cus) * cus);
    };
    // 128-token tiles (64 x 64 wave tiles, a third LDS stage) only where they
    // fill the compute units more than 25% better: on GPT-2 L down (2.5 rounds
    // of 256-token tiles against 5 of 128) the 256-token tiles measured 10%
    // faster over the whole backward (361 -> 325 us)
    return 0.8 * eff(128) > eff(256) ? 128 : 256;
}

size_t dxfold_lds(int BM, const Dims& d) {
    const int nstg = BM == 128 ? 3 : 2;
    return static_cast<size_t>(nstg) * (BM + 4 * 64) * 128 + static_cast<size_t>(d.G) * 4 * 8;
}

bool dxfold_ok(int64_t M, const Dims& d) {
    if (M <= 0 || d.N % 64 != 0 || d.K % 256 != 0 || d.BK % 64 != 0) return false;
    if (static_cast<double>(d.N) * d.Kc * 2.0 >= 2147483648.0) return false;
    if (256.0 * static_cast<double>(d.N) * 2.0 >= 2147483648.0) return false;
    return dxfold_lds(dxfold_bm(M, d), d) <= static_cast<size_t>(max_lds_per_block());
}

template <int BM, int NSTG>
ss1_status launch_dx_fold_cfg(const void* dy, const void* W_c, const int32_t* hash, const int8_t* sign, void* dx,
                              int64_t M, const Dims& d, void* stream) {
    const int n_mt = static_cast<int>((M + BM - 1) / BM);
    const long long blocks = static_cast<long long>(n_mt) * (d.K / 256);
    if (blocks > 0x7FFFFFFFLL) return SS1_ERR_SHAPE;
    const size_t lds = dxfold_lds(BM, d);
    auto kern = &dxfold_kernel<BM, 256, 2, 4, NSTG>;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds)) != hipSuccess)
        return SS1_ERR_HIP;
    hipLaunchKernelGGL((dxfold_kernel<BM, 256, 2, 4, NSTG>), dim3(static_cast<unsigned>(blocks)), dim3(512), lds,
                       static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(dy),
                       static_cast<const uint16_t*>(W_c), hash, sign, static_cast<uint16_t*>(dx), (int)M, (int)d.K,
                       (int)d.N, (int)d.J, (int)d.Jc, d.BK, d.BN, n_mt);
    return hipGetLastError() == hipSuccess ? SS1_OK : SS1_ERR_HIP;
}

}  // namespace

bool fold_supported(const ForwardArgs& a) {
    return a.dtype == SS1_BF16 && fold_config(a).BM > 0;
}

// dW kernel: KT = 256 compressed columns when Kc allows and the c sources fit
// (4*c sub-tiles of 8 KB per stage), else 128; c in {1, 2, 4}; BN % 64 == 0
// (a 64-neuron tile inside one group), BK % 64 == 0; 32-bit buffer offsets
// need x and dy under 2 GiB.
struct DwCfg {
    int KT, NSTG;
    size_t lds;
};

DwCfg dwfold_config(int64_t M, const Dims& d) {
    if (M <= 0 || d.BN % 64 != 0 || d.BK % 64 != 0) return DwCfg{0, 0, 0};
    if (!(d.c == 1 || d.c == 2 || d.c == 4)) return DwCfg{0, 0, 0};
    if (static_cast<double>(M) * std::max(d.K, d.N) * 2.0 >= 2147483648.0) return DwCfg{0, 0, 0};
    int KT = 0;
    if (d.Kc % 256 == 0 && 4 * d.c <= 8) KT = 256;
    else if (d.Kc % 128 == 0 && 2 * d.c <= 8) KT = 128;
    if (KT == 0) return DwCfg{0, 0, 0};
    const size_t stage = static_cast<size_t>(KT / 64 * d.c + 1) * 64 * 128;
    const size_t table = static_cast<size_t>(KT / 64) * (3 * d.c + 1) * 4;
    const size_t cap = static_cast<size_t>(max_lds_per_block());
    int nstg = 3;
    while (nstg > 2 && nstg * stage + table > cap) --nstg;
    // after the loop the stage buffers hold the second half's partial tiles:
    // 4 waves x 16 blocks x 256 floats
    const size_t lds = std::max(nstg * stage + table, static_cast<size_t>(4 * 16 * 256 * 4));
    if (lds > cap) return DwCfg{0, 0, 0};
    return DwCfg{KT, nstg, lds};
}

template <int KT, int CS, int NSTG>
ss1_status launch_dw_fold_cfg(const void* x, const void* dy, const int32_t* hash, const int8_t* sign, void* dW,
                              int64_t M, const Dims& d, const DwCfg& cfg, void* stream) {
    const long long blocks = static_cast<long long>(d.N / 64) * (d.Kc / KT);
    if (blocks > 0x7FFFFFFFLL) return SS1_ERR_SHAPE;
    auto kern = &dwfold_kernel<KT, CS, NSTG>;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(cfg.lds)) != hipSuccess)
        return SS1_ERR_HIP;
    hipLaunchKernelGGL((dwfold_kernel<KT, CS, NSTG>), dim3(static_cast<unsigned>(blocks)), dim3(512), cfg.lds,
                       static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(dy), hash, sign, static_cast<uint16_t*>(dW), (int)M, (int)d.K,
                       (int)d.N, (int)d.J, (int)d.Jc, d.BK, d.BN);
    return hipGetLastError() == hipSuccess ? SS1_OK : SS1_ERR_HIP;
}

template <int KT, int CS>
ss1_status launch_dw_fold_k(const void* x, const void* dy, const int32_t* hash, const int8_t* sign, void* dW,
                            int64_t M, const Dims& d, const DwCfg& cfg, void* stream) {
    if (cfg.NSTG == 3) return launch_dw_fold_cfg<KT, CS, 3>(x, dy, hash, sign, dW, M, d, cfg, stream);
    return launch_dw_fold_cfg<KT, CS, 2>(x, dy, hash, sign, dW, M, d, cfg, stream);
}

bool dx_fold_supported(int64_t M, const Dims& d) { return dxfold_ok(M, d); }

bool dw_fold_supported(int64_t M, const Dims& d) { return dwfold_config(M, d).KT > 0; }

template <int DXBM, int DXNSTG, int KT, int CS, int DWNSTG>
ss1_status launch_bwd_fold_cfg(const void* x, const void* W_c, const int32_t* hash, const int8_t* sign,
                               const void* dy, void* dx, void* dW, int64_t M, const Dims& d, size_t lds,
                               void* stream) {
    const int n_mt = static_cast<int>((M + DXBM - 1) / DXBM);
    const long long n_dw = static_cast<long long>(d.N / 64) * (d.Kc / KT);
    const long long blocks = n_dw + static_cast<long long>(n_mt) * (d.K / 256);
    if (blocks > 0x7FFFFFFFLL) return SS1_ERR_SHAPE;
    auto kern = &bwdfold_kernel<DXBM, DXNSTG, KT, CS, DWNSTG>;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds)) != hipSuccess)
        return SS1_ERR_HIP;
    hipLaunchKernelGGL((bwdfold_kernel<DXBM, DXNSTG, KT, CS, DWNSTG>), dim3(static_cast<unsigned>(blocks)),
                       dim3(512), lds, static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(W_c), hash, sign, static_cast<const uint16_t*>(dy),
                       static_cast<uint16_t*>(dx), static_cast<uint16_t*>(dW), (int)M, (int)d.K, (int)d.N, (int)d.J,
                       (int)d.Jc, d.BK, d.BN, n_mt, static_cast<int>(n_dw));
    return hipGetLastError() == hipSuccess ? SS1_OK : SS1_ERR_HIP;
}

template <int DXBM, int DXNSTG>
ss1_status launch_bwd_fold_dw(const void* x, const void* W_c, const int32_t* hash, const int8_t* sign,
                              const void* dy, void* dx, void* dW, int64_t M, const Dims& d, const DwCfg& cfg,
                              size_t lds, void* stream) {
    // the (KT, c) pairs and the stage counts dwfold_config gives them
    if (cfg.KT == 256 && d.c == 1 && cfg.NSTG == 3)
        return launch_bwd_fold_cfg<DXBM, DXNSTG, 256, 1, 3>(x, W_c, hash, sign, dy, dx, dW, M, d, lds, stream);
    if (cfg.KT == 256 && d.c == 2 && cfg.NSTG == 2)
        return launch_bwd_fold_cfg<DXBM, DXNSTG, 256, 2, 2>(x, W_c, hash, sign, dy, dx, dW, M, d, lds, stream);
    if (cfg.KT == 128 && d.c == 1 && cfg.NSTG == 3)
        return launch_bwd_fold_cfg<DXBM, DXNSTG, 128, 1, 3>(x, W_c, hash, sign, dy, dx, dW, M, d, lds, stream);
    if (cfg.KT == 128 && d.c == 2 && cfg.NSTG == 3)
        return launch_bwd_fold_cfg<DXBM, DXNSTG, 128, 2, 3>(x, W_c, hash, sign, dy, dx, dW, M, d, lds, stream);
    if (cfg.KT == 128 && d.c == 4 && cfg.NSTG == 2)
        return launch_bwd_fold_cfg<DXBM, DXNSTG, 128, 4, 2>(x, W_c, hash, sign, dy, dx, dW, M, d, lds, stream);
    return SS1_ERR_ALGO;
}

bool bwd_fold_supported(int64_t M, const Dims& d) {
    if (!dxfold_ok(M, d)) return false;
    const DwCfg cfg = dwfold_config(M, d);
    if (cfg.KT == 0) return false;
    const size_t lds = std::max(dxfold_lds(dxfold_bm(M, d), d), cfg.lds);
    if (lds > static_cast<size_t>(max_lds_per_block())) return false;
    const bool known = (cfg.KT == 256 && ((d.c == 1 && cfg.NSTG == 3) || (d.c == 2 && cfg.NSTG == 2))) ||
                       (cfg.KT == 128 && ((d.c == 1 && cfg.NSTG == 3) || (d.c == 2 && cfg.NSTG == 3) ||
                                          (d.c == 4 && cfg.NSTG == 2)));
    return known;
}

ss1_status launch_bwd_fold(const void* x, const void* W_c, const int32_t* hash, const int8_t* sign, const void* dy,
                           void* dx, void* dW, int64_t M, const Dims& d, void* stream) {
    if (!bwd_fold_supported(M, d)) return SS1_ERR_ALGO;
    const DwCfg cfg = dwfold_config(M, d);
    const int bm = dxfold_bm(M, d);
    const size_t lds = std::max(dxfold_lds(bm, d), cfg.lds);
    if (bm == 128) return launch_bwd_fold_dw<128, 3>(x, W_c, hash, sign, dy, dx, dW, M, d, cfg, lds, stream);
    return launch_bwd_fold_dw<256, 2>(x, W_c, hash, sign, dy, dx, dW, M, d, cfg, lds, stream);
}

ss1_status launch_dw_fold(const void* x, const void* dy, const int32_t* hash, const int8_t* sign, void* dW,
                          int64_t M, const Dims& d, void* stream) {
    const DwCfg cfg = dwfold_config(M, d);
    if (cfg.KT == 256) {
        if (d.c == 1) return launch_dw_fold_k<256, 1>(x, dy, hash, sign, dW, M, d, cfg, stream);
        if (d.c == 2) return launch_dw_fold_k<256, 2>(x, dy, hash, sign, dW, M, d, cfg, stream);
    }
    if (cfg.KT == 128) {
        if (d.c == 1) return launch_dw_fold_k<128, 1>(x, dy, hash, sign, dW, M, d, cfg, stream);
        if (d.c == 2) return launch_dw_fold_k<128, 2>(x, dy, hash, sign, dW, M, d, cfg, stream);
        if (d.c == 4) return launch_dw_fold_k<128, 4>(x, dy, hash, sign, dW, M, d, cfg, stream);
    }
    return SS1_ERR_ALGO;
}

ss1_status launch_dx_fold(const void* dy, const void* W_c, const int32_t* hash, const int8_t* sign, void* dx,
                          int64_t M, const Dims& d, void* stream) {
    if (!dxfold_ok(M, d)) return SS1_ERR_ALGO;
    if (dxfold_bm(M, d) == 128) return launch_dx_fold_cfg<128, 3>(dy, W_c, hash, sign, dx, M, d, stream);
    return launch_dx_fold_cfg<256, 2>(dy, W_c, hash, sign, dx, M, d, stream);
}

// Run time model fitted to MI355X measurements of the 256 x 256 tile (inputs
// not in cache): per round of tiles (one tile per compute unit) 31 ns per
// input element of K plus 10 us; the 4-wave tiles run about 1.3x slower per
// unit of area, and a round of the 128 x 256 tiles of a split launch takes
// 0.55 of a full one.
double fold_estimate_us(const ForwardArgs& a) {
    const FoldCfg cfg = fold_config(a);
    if (a.dtype != SS1_BF16 || cfg.BM == 0 || a.M <= 0) return 1e300;
    const double cus = device_attribute(hipDeviceAttributeMultiprocessorCount, 256);
    const double per_round = 0.031 * static_cast<double>(a.d.K) + 10.0;
    const int64_t main = fold_main_cols(a, cfg);
    const double n_mt = std::ceil(static_cast<double>(a.M) / cfg.BM);
    if (main != a.d.N) {
        const double t_main = std::ceil(n_mt * static_cast<double>(main / 256) / cus);
        const double t_rest = std::ceil(std::ceil(static_cast<double>(a.M) / 128) *
                                        static_cast<double>((a.d.N - main) / 256) / cus);
        return (t_main + 0.55 * t_rest) * per_round;
    }
    const double tiles = n_mt * static_cast<double>(a.d.N / cfg.BNB);
    const double rounds = std::ceil(tiles / cus);
    const double area = static_cast<double>(cfg.BM) * cfg.BNB / 65536.0;
    // tiles 128 neurons wide run 4 waves (or 64 x 64 wave tiles), about 1.3x
    // the time per unit of area of the 8-wave tiles 256 neurons wide
    return rounds * per_round * area * (cfg.BNB < 256 ? 1.3 : 1.0);
}

ss1_status launch_fold(const ForwardArgs& a) {
    // fp8 weights come with the forward hash only
    if (a.w_fp8) return a.form == PlanForm::Hash ? launch_fold_t<true, true>(a) : SS1_ERR_ALGO;
    return a.form == PlanForm::Hash ? launch_fold_t<true, false>(a) : launch_fold_t<false, false>(a);
}

// fp8 fold (both operands E4M3): 256 x 256 tiles, two 64 KB stages.  Needs
// N a multiple of 256 split into whole groups, BK % 64 == 0 (each 64-input
// weight half inside one chunk), K % 128 == 0, and 32-bit byte offsets over a
// tile's x rows and over W_c.
size_t fold8_lds(const Dims& d) { return static_cast<size_t>(2) * 64 * 1024 + static_cast<size_t>(256 / d.BN) * d.J * 8; }

bool fold8_supported(int64_t M, const Dims& d) {
    if (M < 0 || d.N % 256 != 0 || 256 % d.BN != 0 || d.BK % 64 != 0 || d.K % 128 != 0) return false;
    if (256.0 * static_cast<double>(d.K) >= 2147483648.0 || static_cast<double>(d.N) * d.Kc >= 2147483648.0) return false;
    return fold8_lds(d) <= static_cast<size_t>(max_lds_per_block());
}

ss1_status launch_fold8(const void* xq, const float* xs, const void* wq, const float* ws, const int32_t* hash,
                        const int8_t* sign, void* y, int64_t M, const Dims& d, int32_t act, void* stream) {
    if (!fold8_supported(M, d)) return SS1_ERR_ALGO;
    if (M == 0) return SS1_OK;
    const int n_mt = static_cast<int>((M + 255) / 256);
    const long long blocks = static_cast<long long>(n_mt) * (d.N / 256);
    if (blocks > 0x7FFFFFFFLL) return SS1_ERR_SHAPE;
    const size_t lds = fold8_lds(d);
    auto kern = &fold8_kernel<2>;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds)) != hipSuccess)
        return SS1_ERR_HIP;
    hipLaunchKernelGGL((fold8_kernel<2>), dim3(static_cast<unsigned>(blocks)), dim3(512), lds,
                       static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(xq), xs,
                       static_cast<const uint8_t*>(wq), ws, hash, sign, static_cast<uint16_t*>(y), (int)M, (int)d.K,
                       (int)d.N, (int)d.J, (int)d.Jc, d.BK, d.BN, n_mt, act);
    return hipGetLastError() == hipSuccess ? SS1_OK : SS1_ERR_HIP;
}

}  // namespace ss1
