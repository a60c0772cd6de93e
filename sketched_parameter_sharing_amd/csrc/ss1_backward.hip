// Backward of the SS1 forward (the SS1 summary page, "Limitations": the
// backward pass is not reduced).  With y[:, g-block] = z_g W_c[g-block]^T:
//   dW_c[g-block] = dy[:, g-block]^T z_g                    (dw_kernel)
//   dx[:, j-chunk] = sum_g sign[g][j] (dy[:, g-block] W_c[g-block])[:, hash[g][j]-chunk]
//                  = dy times the dense expansion of W_c          (dx_kernel)
// Both run on 16x16x32 bf16 MFMA with float32 accumulation.  Where their
// shape conditions hold, both go to the fold kernels of ss1_fold.hip instead
// (no sketch formed; dense MFMA work): dW_c when BN % 64 == 0, BK % 64 == 0,
// c in {1, 2, 4} and Kc % 128 == 0; dx when N % 64 == 0, K % 256 == 0 and
// BK % 64 == 0.  The operands
// whose stored rows run along the reduction dimension are written to LDS as
// stored (16-byte stores) and read back transposed with ds_read_b64_tr_b16.
//
// dw_kernel: block = 4 waves, output tile 32 neurons (inside one group) x 32
//   or 128 compressed columns; wave w reduces over its quarter of the tokens.
//   Per chunk of 64 (or 32) tokens the wave writes its dy tile and sketch tile
//   into LDS (the sketch summed in float32 over the c sources in
//   ascending order and rounded to bf16, as in the forward) and runs its
//   MFMAs on them; the four partial tiles are summed at the end.
// dx: the fold kernel's dx variant (ss1_fold.hip) when N % 64 == 0, K % 256
//   == 0 and BK % 64 == 0; otherwise
// dx_wide_kernel (K % 128 == 0, N % 64 == 0): 128 x 128 dx tiles, see below.
// dx_kernel (otherwise): block = 4 waves, output tile 128 tokens x 32 columns of one input
//   chunk j, wave w owning tokens [32w, 32w+32).  Per stage of 128 neurons
//   (32 when N is not a multiple of 128) the block stages, for each neuron of
//   group g, its W_c columns of compressed chunk hash[g][j] with sign[g][j] on
//   the sign bits (the chunk's target and sign per group sit in an LDS table);
//   dy is read straight into the MFMA operand (its rows are contiguous along
//   n).  Stages are double-buffered: the loads of stage s+1 travel while the
//   MFMAs of stage s run, one barrier per stage.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "ss1_device.h"
#include "ss1_internal.h"

namespace ss1 {

namespace {

using namespace dev;

constexpr int kDwN = 32;           // neurons per dw block
constexpr int kDwPN = kDwN + 8;    // LDS pitch of the dy tile (elements)

// Block: 4 waves on one 32 x KT output tile (KT = 32 or 128 compressed
// columns, inside one compressed chunk when KT <= BK), wave w reducing over
// its quarter of the tokens with tiles of its own in LDS (no block barrier
// inside the loop); the four partial sums meet in LDS at the end.
template <int C_T, int KT>
__global__ __launch_bounds__(256) void dw_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ dy,
                                                 const int32_t* __restrict__ pi, const int8_t* __restrict__ ps,
                                                 uint16_t* __restrict__ dw, int M, int K, int N, int J, int Jc,
                                                 int c_rt, int BK, int BN) {
    constexpr int MC = KT == 32 ? 64 : 32;   // tokens per chunk of one wave
    constexpr int PK = KT + 8;               // LDS pitch of the sketch tile
    constexpr int TILE = MC * (kDwPN + PK);  // elements per wave
    constexpr int NB = KT / 16;              // 16-column blocks per wave
    __shared__ __align__(16) uint16_t tiles[4 * TILE];
    extern __shared__ uint32_t smem[];
    uint32_t* s_src = smem;
    int* s_cnt = reinterpret_cast<int*>(smem + J);

    const int c = (C_T > 0) ? C_T : c_rt;
    const int Kc = Jc * BK;
    const int tiles_per_group = BN / kDwN;
    const int g = blockIdx.x / tiles_per_group;
    const int n0 = g * BN + (blockIdx.x % tiles_per_group) * kDwN;
    const int k0 = blockIdx.y * KT;
    stage_plan<true>(pi, ps, g, J, Jc, c, BK, s_src, s_cnt);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    uint16_t* DY = tiles + wave * TILE;
    uint16_t* Z = DY + MC * kDwPN;
    const int mq = (M + 3) / 4;                       // tokens per wave
    const int mb = wave * mq;
    const int me = min(M, mb + mq);

    f32x4 acc[2][NB];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    for (int m0 = mb; m0 < me; m0 += MC) {
        // dy: lane -> token lane/4 + 16*i, neurons 8*(lane%4) .. +7
#pragma unroll
        for (int i = 0; i < MC / 16; ++i) {
            const int mm = (lane >> 2) + 16 * i;
            const int c8 = (lane & 3) * 8;
            uint4 dv = make_uint4(0, 0, 0, 0);
            if (m0 + mm < me) dv = *reinterpret_cast<const uint4*>(dy + static_cast<size_t>(m0 + mm) * N + n0 + c8);
            *reinterpret_cast<uint4*>(DY + mm * kDwPN + c8) = dv;
        }
        // sketch: lane -> token lane/(KT/8) + (512/KT)*i, columns k0 + 8*(lane%(KT/8)) .. +7
        constexpr int LPR = KT / 8;        // lanes per token row
        constexpr int RPI = 64 / LPR;      // token rows per pass
#pragma unroll
        for (int i = 0; i < MC / RPI; ++i) {
            const int mm = lane / LPR + RPI * i;
            const int kk = (lane % LPR) * 8;
            const int kp = k0 + kk;
            uint4 zv = make_uint4(0, 0, 0, 0);
            if (m0 + mm < me) {
                const int t = kp / BK;
                const int u = kp - t * BK;
                const uint16_t* xr = x + static_cast<size_t>(m0 + mm) * K + u;
                float sm[8];
                if constexpr (C_T > 0) {
                    uint4 raw[C_T];
#pragma unroll
                    for (int r = 0; r < C_T; ++r)
                        raw[r] = *reinterpret_cast<const uint4*>(xr + (s_src[t * C_T + r] & kOffMask));
#pragma unroll
                    for (int r = 0; r < C_T; ++r) {
                        const uint32_t e = s_src[t * C_T + r];
                        acc_sign8(sm, raw[r], entry_sign(e), entry_sign_xor(e), r == 0);
                    }
                } else {
                    for (int r = 0; r < c; ++r) {
                        const uint32_t e = s_src[t * c + r];
                        const uint4 raw = *reinterpret_cast<const uint4*>(xr + (e & kOffMask));
                        acc_sign8(sm, raw, entry_sign(e), entry_sign_xor(e), r == 0);
                    }
                }
                zv = pack_bf16x8(sm);
            }
            *reinterpret_cast<uint4*>(Z + mm * PK + kk) = zv;
        }
        // the wave's own tiles: its LDS writes must land before its reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
        for (int ks = 0; ks < MC; ks += 32) {
            bf16x8 af[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) af[a] = lds_operand_tr(DY, kDwPN, ks, 16 * a, lane);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const bf16x8 bfr = lds_operand_tr(Z, PK, ks, 16 * b, lane);
#pragma unroll
                for (int a = 0; a < 2; ++a)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bfr, acc[a][b], 0, 0, 0);
            }
        }
        // the next chunk overwrites the tiles only after these reads completed
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    }
    // sum the four waves' partial tiles (fixed order: wave 0 + 1 + 2 + 3), one
    // 16-column block at a time through the (now free) tile memory
    float* red = reinterpret_cast<float*>(tiles);   // [3][8][64] floats per column block
    static_assert(3 * 8 * 64 * 4 <= 4 * TILE * 2, "reduction buffer");
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        __syncthreads();
        if (wave > 0) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int q = 0; q < 4; ++q) red[((wave - 1) * 8 + a * 4 + q) * 64 + lane] = acc[a][b][q];
        }
        __syncthreads();
        if (wave == 0) {
            const int col = k0 + 16 * b + (lane & 15);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float v = acc[a][b][q];
#pragma unroll
                    for (int w = 0; w < 3; ++w) v += red[(w * 8 + a * 4 + q) * 64 + lane];
                    const int n = n0 + 16 * a + (lane >> 4) * 4 + q;
                    dw[static_cast<size_t>(n) * Kc + col] = to_bf16_bits(v);
                }
        }
    }
}

constexpr int kDxM = 128;       // tokens per dx block
constexpr int kDxU = 32;        // columns per dx block (inside one input chunk)
constexpr int kDxPU = kDxU + 8; // LDS pitch of the staged W_c slice (elements)

// NS neurons staged per barrier (128, or 32 when N is not a multiple of 128).
// Dynamic LDS: one word per group, the target chunk's column offset and sign.
template <int NS>
__global__ __launch_bounds__(256) void dx_kernel(const uint16_t* __restrict__ dy, const uint16_t* __restrict__ w,
                                                 const int32_t* __restrict__ pi, const int8_t* __restrict__ ps,
                                                 uint16_t* __restrict__ dx, int M, int K, int N, int J, int Jc,
                                                 int BK, int BN) {
    __shared__ __align__(16) uint16_t WS[2][NS * kDxPU];   // signed W_c slices, row n, double-buffered
    extern __shared__ uint32_t gtab[];
    const int Kc = Jc * BK;
    const int G = N / BN;
    const int m0 = blockIdx.x * kDxM;
    const int col0 = blockIdx.y * kDxU;   // dx columns [col0, col0 + 32)
    const int j = col0 / BK;
    const int uoff = col0 - j * BK;

    const int tid = threadIdx.x;
    for (int g = tid; g < G; g += 256) {
        const int t = pi[static_cast<size_t>(g) * J + j];
        gtab[g] = static_cast<uint32_t>(t * BK) | (ps[static_cast<size_t>(g) * J + j] < 0 ? kNeg : 0u);
    }
    __syncthreads();

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
    constexpr int KS = NS / 32;              // MFMA k-steps per stage
    constexpr int WV = (NS * 4 + 255) / 256; // W vectors per thread per stage
    const int nstage = N / NS;

    struct Regs {
        bf16x8 af[KS][2];
        uint4 wv[WV];
    };
    auto issue = [&](int st, Regs& R) {
        const int nb = min(st, nstage - 1) * NS;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int a = 0; a < 2; ++a) R.af[kk][a] = *reinterpret_cast<const bf16x8*>(dyr[a] + nb + 32 * kk);
#pragma unroll
        for (int i = 0; i < WV; ++i) {
            const int v = min(tid + i * 256, NS * 4 - 1);
            const int n = nb + (v >> 2);
            const uint32_t e = gtab[n / BN];
            uint4 val = *reinterpret_cast<const uint4*>(w + static_cast<size_t>(n) * Kc + (e & kOffMask) + uoff +
                                                         (v & 3) * 8);
            const uint32_t flip = (e & kNeg) ? 0x80008000u : 0u;
            val.x ^= flip;
            val.y ^= flip;
            val.z ^= flip;
            val.w ^= flip;
            R.wv[i] = val;
        }
    };
    auto commit = [&](const Regs& R, int buf) {
#pragma unroll
        for (int i = 0; i < WV; ++i) {
            const int v = tid + i * 256;
            if (v < NS * 4) *reinterpret_cast<uint4*>(&WS[buf][(v >> 2) * kDxPU + (v & 3) * 8]) = R.wv[i];
        }
    };

    f32x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    Regs cur, nxt;
    issue(0, cur);
    commit(cur, 0);
    __syncthreads();
    for (int st = 0; st < nstage; ++st) {
        issue(st + 1, nxt);   // past the last stage this re-reads it; never used
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            bf16x8 bfr[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) bfr[b] = lds_operand_tr(WS[st & 1], kDxPU, 32 * kk, 16 * b, lane);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.af[kk][a], bfr[b], acc[a][b], 0, 0, 0);
        }
        commit(nxt, (st + 1) & 1);
        cur = nxt;
        __syncthreads();
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

// Wide dx tile: block = 2 x 2 waves on 128 tokens x 128 dx columns (columns
// [col0, col0 + 128), spanning 128/BK input chunks or lying inside one), wave
// (wm, wu) owning 64 x 64.  Per stage of 64 neurons the block stages the
// signed W_c columns each neuron's group maps the tile's chunks to (double
// buffered, one barrier per stage); the dy operands of the next stage are
// requested before the current stage's MFMAs.  Dynamic LDS: per group g and
// chunk jj of the tile, the target's column offset and sign.
constexpr int kDxwT = 128;             // tokens and columns per block
constexpr int kDxwN = 64;              // neurons per stage
constexpr int kDxwP = kDxwT + 8;       // LDS pitch (elements)

__global__ __launch_bounds__(256) void dx_wide_kernel(const uint16_t* __restrict__ dy, const uint16_t* __restrict__ w,
                                                      const int32_t* __restrict__ pi, const int8_t* __restrict__ ps,
                                                      uint16_t* __restrict__ dx, int M, int K, int N, int J, int Jc,
                                                      int BK, int BN) {
    __shared__ __align__(16) uint16_t WS[2][kDxwN * kDxwP];
    extern __shared__ uint32_t gtab[];
    const int Kc = Jc * BK;
    const int G = N / BN;
    const int m0 = blockIdx.x * kDxwT;
    const int col0 = blockIdx.y * kDxwT;
    const int j0 = col0 / BK;
    // chunks a 128-column window on 32-column boundaries can touch (BK % 32 == 0)
    const int cpt = (kDxwT - 32) / BK + 2;
    const int tid = threadIdx.x;
    for (int e = tid; e < G * cpt; e += 256) {
        const int g = e / cpt;
        const int j = j0 + e % cpt;
        gtab[e] = 0;
        if (j < J) {
            const int t = pi[static_cast<size_t>(g) * J + j];
            gtab[e] = static_cast<uint32_t>(t * BK) | (ps[static_cast<size_t>(g) * J + j] < 0 ? kNeg : 0u);
        }
    }
    __syncthreads();

    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wu = wave & 1;
    const int fr = lane & 15;
    const int fk = (lane >> 4) * 8;
    const uint16_t* dyr[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int m = min(m0 + wm * 64 + 16 * a + fr, M - 1);   // rows past M are never stored
        dyr[a] = dy + static_cast<size_t>(m) * N + fk;
    }
    const int nstage = N / kDxwN;

    struct Regs {
        bf16x8 af[2][4];   // [k-step][m block]
        uint4 wv[4];
    };
    auto issue = [&](int st, Regs& R) {
        const int nb = min(st, nstage - 1) * kDxwN;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int a = 0; a < 4; ++a) R.af[kk][a] = *reinterpret_cast<const bf16x8*>(dyr[a] + nb + 32 * kk);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int v = tid + i * 256;           // 64 neurons x 16 vectors
            const int n = nb + (v >> 4);
            const int col = col0 + (v & 15) * 8;
            const int j = col / BK;
            const uint32_t e = gtab[(n / BN) * cpt + (j - j0)];
            uint4 val = *reinterpret_cast<const uint4*>(w + static_cast<size_t>(n) * Kc + (e & kOffMask) +
                                                         (col - j * BK));
            const uint32_t flip = (e & kNeg) ? 0x80008000u : 0u;
            val.x ^= flip;
            val.y ^= flip;
            val.z ^= flip;
            val.w ^= flip;
            R.wv[i] = val;
        }
    };
    auto commit = [&](const Regs& R, int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int v = tid + i * 256;
            *reinterpret_cast<uint4*>(&WS[buf][(v >> 4) * kDxwP + (v & 15) * 8]) = R.wv[i];
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    Regs cur, nxt;
    issue(0, cur);
    commit(cur, 0);
    __syncthreads();
    for (int st = 0; st < nstage; ++st) {
        issue(st + 1, nxt);   // past the last stage this re-reads it; never used
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const bf16x8 bfr = lds_operand_tr(WS[st & 1], kDxwP, 32 * kk, wu * 64 + 16 * b, lane);
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.af[kk][a], bfr, acc[a][b], 0, 0, 0);
            }
        }
        commit(nxt, (st + 1) & 1);
        cur = nxt;
        __syncthreads();
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int col = col0 + wu * 64 + 16 * b + fr;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = m0 + wm * 64 + 16 * a + (lane >> 4) * 4 + q;
                if (m < M) dx[static_cast<size_t>(m) * K + col] = to_bf16_bits(acc[a][b][q]);
            }
        }
}

template <int C_T, int KT>
ss1_status launch_dw_kt(const void* x, const void* dy, const int32_t* hash, const int8_t* sign, void* dW,
                        int64_t M, const Dims& d, void* stream) {
    const dim3 grid(static_cast<unsigned>(d.G * (d.BN / kDwN)), static_cast<unsigned>(d.Kc / KT));
    const size_t lds = static_cast<size_t>(d.J + d.Jc) * 4;
    hipLaunchKernelGGL((dw_kernel<C_T, KT>), grid, dim3(256), lds, static_cast<hipStream_t>(stream),
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(dy), hash, sign,
                       static_cast<uint16_t*>(dW), (int)M, (int)d.K, (int)d.N, (int)d.J, (int)d.Jc, d.c, d.BK,
                       d.BN);
    return hipGetLastError() == hipSuccess ? SS1_OK : SS1_ERR_HIP;
}

// 128-column tiles for wide layers (fewer re-reads of dy), 32 otherwise (more
// blocks for narrow ones)
template <int C_T>
ss1_status launch_dw_cfg(const void* x, const void* dy, const int32_t* hash, const int8_t* sign, void* dW,
                         int64_t M, const Dims& d, void* stream) {
    if (d.Kc >= 1024 && d.Kc % 128 == 0) return launch_dw_kt<C_T, 128>(x, dy, hash, sign, dW, M, d, stream);
    return launch_dw_kt<C_T, 32>(x, dy, hash, sign, dW, M, d, stream);
}

}  // namespace

ss1_status launch_backward(const void* x, const void* W_c, const int32_t* hash, const int8_t* sign, const void* dy,
                           void* dx, void* dW, int64_t M, const Dims& d, void* stream) {
    if (dx && dW && M > 0 && bwd_fold_supported(M, d))
        return launch_bwd_fold(x, W_c, hash, sign, dy, dx, dW, M, d, stream);
    if (dW && dw_fold_supported(M, d)) {
        const ss1_status st = launch_dw_fold(x, dy, hash, sign, dW, M, d, stream);
        if (st != SS1_OK) return st;
    } else if (dW) {
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
        if (dx_fold_supported(M, d)) return launch_dx_fold(dy, W_c, hash, sign, dx, M, d, stream);
        const int cpt = static_cast<int>((kDxwT - 32) / d.BK + 2);
        if (d.K % kDxwT == 0 && d.N % kDxwN == 0 && d.G * cpt <= 8192) {
            const dim3 grid(static_cast<unsigned>((M + kDxwT - 1) / kDxwT), static_cast<unsigned>(d.K / kDxwT));
            const size_t lds = static_cast<size_t>(d.G) * cpt * 4;
            hipLaunchKernelGGL(dx_wide_kernel, grid, dim3(256), lds, static_cast<hipStream_t>(stream),
                               static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(W_c), hash, sign,
                               static_cast<uint16_t*>(dx), (int)M, (int)d.K, (int)d.N, (int)d.J, (int)d.Jc, d.BK,
                               d.BN);
            return hipGetLastError() == hipSuccess ? SS1_OK : SS1_ERR_HIP;
        }
        const dim3 grid(static_cast<unsigned>((M + kDxM - 1) / kDxM), static_cast<unsigned>(d.K / kDxU));
        const size_t lds = static_cast<size_t>(d.G) * 4;   // G <= 8192 (checked by the caller)
        if (d.N % 128 == 0)
            hipLaunchKernelGGL((dx_kernel<128>), grid, dim3(256), lds, static_cast<hipStream_t>(stream),
                               static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(W_c), hash, sign,
                               static_cast<uint16_t*>(dx), (int)M, (int)d.K, (int)d.N, (int)d.J, (int)d.Jc, d.BK,
                               d.BN);
        else
            hipLaunchKernelGGL((dx_kernel<32>), grid, dim3(256), lds, static_cast<hipStream_t>(stream),
                               static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(W_c), hash, sign,
                               static_cast<uint16_t*>(dx), (int)M, (int)d.K, (int)d.N, (int)d.J, (int)d.Jc, d.BK,
                               d.BN);
        if (hipGetLastError() != hipSuccess) return SS1_ERR_HIP;
    }
    return SS1_OK;
}

}  // namespace ss1
