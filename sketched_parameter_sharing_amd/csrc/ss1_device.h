// Device-side building blocks shared by the SS1 kernels: the plan as kept in
// LDS, bf16 conversions, the signed sketch accumulation, buffer-resource
// loads, operand permutes and the XCD-aware tile order.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "ss1_internal.h"

namespace ss1 {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Workgroup barrier that orders LDS only: global loads still in flight stay in
// flight (a plain __syncthreads also waits for them).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Buffer-resource loads: a scalar base (the descriptor) plus a per-lane 32-bit
// byte offset and a scalar byte offset, so per-step addressing costs no vector
// instructions.  Reads at or past `bytes` return zero.
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit data format, gfx9 family
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kBufferWord3);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// ---------------------------------------------------------------- plan in LDS
// One 32-bit word per source: element offset of the source chunk inside an x
// row (bits 0..29), "negative" (bit 31), "absent" (bit 30).
constexpr uint32_t kNeg = 0x80000000u;
constexpr uint32_t kAbsent = 0x40000000u;
constexpr uint32_t kOffMask = 0x3FFFFFFFu;

__device__ __forceinline__ float entry_sign(uint32_t e) {
    return (e & kAbsent) ? 0.0f : __uint_as_float((e & kNeg) | 0x3F800000u);
}

__device__ __forceinline__ uint32_t make_entry(int j, int BK, int s) {
    return static_cast<uint32_t>(j * BK) | (s < 0 ? kNeg : 0u);
}

// Fills s_src[t*c + r] (t < Jc, r < c) for group g.  From the forward hash the
// sources of each compressed chunk are gathered with LDS atomics and then put
// in ascending chunk order; from the inverse index they are copied.  Needs
// s_cnt[Jc] scratch for the forward form.  Ends with a barrier.  The
// barriers order LDS only: global loads issued before the call stay in flight.
template <bool FROM_HASH>
__device__ void stage_plan(const int32_t* __restrict__ pi, const int8_t* __restrict__ ps, int g,
                           int J, int Jc, int c, int BK, uint32_t* s_src, int* s_cnt) {
    const int tid = threadIdx.x;
    const int nt = blockDim.x;
    const int32_t* gi = pi + static_cast<size_t>(g) * J;
    const int8_t* gs = ps + static_cast<size_t>(g) * J;
    if (FROM_HASH) {
        for (int e = tid; e < J; e += nt) s_src[e] = kAbsent;
        for (int t = tid; t < Jc; t += nt) s_cnt[t] = 0;
        lds_barrier();
        for (int j = tid; j < J; j += nt) {
            const int t = gi[j];
            const int s = gs[j];
            if (t >= 0 && t < Jc && (s == 1 || s == -1)) {
                const int slot = atomicAdd(&s_cnt[t], 1);
                if (slot < c) s_src[t * c + slot] = make_entry(j, BK, s);
            }
        }
        lds_barrier();
        for (int t = tid; t < Jc; t += nt) {
            uint32_t* p = s_src + t * c;
            for (int a = 1; a < c; ++a) {  // insertion sort; absent entries go last
                const uint32_t v = p[a];
                int b = a - 1;
                while (b >= 0 && (p[b] & ~kNeg) > (v & ~kNeg)) {
                    p[b + 1] = p[b];
                    --b;
                }
                p[b + 1] = v;
            }
        }
    } else {
        for (int e = tid; e < J; e += nt) {
            const int j = gi[e];
            const int s = gs[e];
            s_src[e] = (j >= 0 && j < J && (s == 1 || s == -1)) ? make_entry(j, BK, s) : kAbsent;
        }
    }
    lds_barrier();
}

// Buffer loads with the hardware range check: an offset at or past the
// descriptor's extent reads zeros and moves no data, so the loads need no
// branches (a branch around a load makes the compiler wait for it at the join).
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
}
__device__ __forceinline__ int8_t buf_load1(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return static_cast<int8_t>(__builtin_amdgcn_raw_buffer_load_b8(r, voff, 0, 0));
}
constexpr uint32_t kOutOfRange = 0x80000000u;  // past every extent used here

// Cache policy of the weight loads: non-temporal (each weight is read once;
// measured about 5% faster on the Llama-3-8B decode shapes than the default).
constexpr int kNonTemporal = 2;

// Plan entries per thread when each thread reads its entries of the group's
// plan into registers itself (stage_plan_regs): J <= 2 * threads.
constexpr int kPlanPerThread = 2;

// Reads this thread's entries j = tid + p * blockDim.x (p < PJ) of group g's
// plan into registers, as branch-free buffer loads (zeros past J).
template <int PJ>
__device__ __forceinline__ void fetch_plan_regs(const int32_t* __restrict__ pi, const int8_t* __restrict__ ps,
                                                int g, int J, int32_t (&iv)[PJ], int8_t (&sv)[PJ]) {
    const __amdgpu_buffer_rsrc_t prs = make_rsrc(pi + static_cast<size_t>(g) * J, static_cast<uint32_t>(J) * 4);
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(ps + static_cast<size_t>(g) * J, static_cast<uint32_t>(J));
#pragma unroll
    for (int p = 0; p < PJ; ++p) {
        const uint32_t j = static_cast<uint32_t>(threadIdx.x + p * blockDim.x);
        iv[p] = static_cast<int32_t>(buf_load4(prs, 4 * j));
        sv[p] = buf_load1(srs, j);
    }
}

// Stages the plan of group g (as stage_plan does) from entries that each
// thread has already read into registers: entry j = tid + p * nt is iv[p],
// sv[p] (entries at j >= J are ignored).  Ends with a barrier that orders LDS
// only.
template <bool FROM_HASH, int PJ>
__device__ void stage_plan_regs(const int32_t (&iv)[PJ], const int8_t (&sv)[PJ], int J, int Jc, int c, int BK,
                                uint32_t* s_src, int* s_cnt) {
    const int tid = threadIdx.x;
    const int NT = blockDim.x;
    if (FROM_HASH) {
        for (int e = tid; e < J; e += NT) s_src[e] = kAbsent;
        for (int t = tid; t < Jc; t += NT) s_cnt[t] = 0;
        lds_barrier();
#pragma unroll
        for (int p = 0; p < PJ; ++p) {
            const int j = tid + p * NT;
            const int t = iv[p];
            const int s = sv[p];
            if (j < J && t >= 0 && t < Jc && (s == 1 || s == -1)) {
                const int slot = atomicAdd(&s_cnt[t], 1);
                if (slot < c) s_src[t * c + slot] = make_entry(j, BK, s);
            }
        }
        lds_barrier();
        for (int t = tid; t < Jc; t += NT) {
            uint32_t* p = s_src + t * c;
            for (int a = 1; a < c; ++a) {  // ascending source chunk; absent entries last
                const uint32_t v = p[a];
                int b = a - 1;
                while (b >= 0 && (p[b] & ~kNeg) > (v & ~kNeg)) {
                    p[b + 1] = p[b];
                    --b;
                }
                p[b + 1] = v;
            }
        }
    } else {
#pragma unroll
        for (int p = 0; p < PJ; ++p) {
            const int e = tid + p * NT;
            const int j = iv[p];
            const int s = sv[p];
            if (e < J) s_src[e] = (j >= 0 && j < J && (s == 1 || s == -1)) ? make_entry(j, BK, s) : kAbsent;
        }
    }
    lds_barrier();
}

// ------------------------------------------------------------- bf16 helpers
// A 32-bit word holding two bf16 values (element 2i in the low half): their
// float32 values are the halves moved to the top of a word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two float32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float round_to_bf16(float v) {
    return __uint_as_float(pack_bf16(v, 0.0f) << 16);
}

__device__ __forceinline__ uint16_t to_bf16_bits(float v) {
    return static_cast<uint16_t>(pack_bf16(v, 0.0f) & 0xFFFFu);
}

// Accumulates one 16-byte vector of 8 bf16 into acc[8] (first source sets it).
__device__ __forceinline__ void acc_bf16x8(float (&acc)[8], const uint4& raw, float s, bool first) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = bf16_lo(w[i]);
        const float hi = bf16_hi(w[i]);
        if (first) {
            acc[2 * i] = s * lo;
            acc[2 * i + 1] = s * hi;
        } else {
            acc[2 * i] = fmaf(s, lo, acc[2 * i]);
            acc[2 * i + 1] = fmaf(s, hi, acc[2 * i + 1]);
        }
    }
}

__device__ __forceinline__ uint4 pack_bf16x8(const float (&acc)[8]) {
    uint4 r;
    r.x = pack_bf16(acc[0], acc[1]);
    r.y = pack_bf16(acc[2], acc[3]);
    r.z = pack_bf16(acc[4], acc[5]);
    r.w = pack_bf16(acc[6], acc[7]);
    return r;
}

// Sketch of 8 consecutive elements from one more signed source, in float32.
// The first source is exact: its sign goes onto the bf16 sign bits (sgnx,
// 0x80008000 or 0) before the halves are widened.  Each further source is
// widened and added with a fused multiply-add by its sign (+-1.0, or 0 for a
// source a malformed plan leaves absent), one float32 rounding per add, in
// source order.  On gfx950 these integer and FMA instructions issue alongside
// the MFMAs of other waves; the bf16 dot-product instructions do not, which is
// why they are not used here.
__device__ __forceinline__ void acc_sign8(float (&acc)[8], const uint4& raw, float sgn, uint32_t sgnx,
                                          bool first) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (first) {
            const uint32_t v = w[i] ^ sgnx;
            acc[2 * i] = bf16_lo(v);
            acc[2 * i + 1] = bf16_hi(v);
        } else {
            acc[2 * i] = fmaf(sgn, bf16_lo(w[i]), acc[2 * i]);
            acc[2 * i + 1] = fmaf(sgn, bf16_hi(w[i]), acc[2 * i + 1]);
        }
    }
}

// Sign of a plan entry as a mask on a pair of bf16 values.
__device__ __forceinline__ uint32_t entry_sign_xor(uint32_t e) {
    return (e & kNeg) ? 0x80008000u : 0u;
}

// Plans of `count` consecutive groups starting at g0, one J-entry row per
// group in s_src (same encoding as stage_plan).  s_cnt needs count*Jc ints in
// the forward form.  Ends with a barrier.
template <bool FROM_HASH>
__device__ void stage_plans(const int32_t* __restrict__ pi, const int8_t* __restrict__ ps, int g0,
                            int count, int J, int Jc, int c, int BK, uint32_t* s_src, int* s_cnt) {
    const int tid = threadIdx.x;
    const int nt = blockDim.x;
    const int total = count * J;
    const int32_t* gi = pi + static_cast<size_t>(g0) * J;
    const int8_t* gs = ps + static_cast<size_t>(g0) * J;
    if (FROM_HASH) {
        for (int e = tid; e < total; e += nt) s_src[e] = kAbsent;
        for (int e = tid; e < count * Jc; e += nt) s_cnt[e] = 0;
        lds_barrier();
        for (int e = tid; e < total; e += nt) {
            const int gl = e / J;
            const int j = e - gl * J;
            const int t = gi[e];
            const int s = gs[e];
            if (t >= 0 && t < Jc && (s == 1 || s == -1)) {
                const int slot = atomicAdd(&s_cnt[gl * Jc + t], 1);
                if (slot < c) s_src[gl * J + t * c + slot] = make_entry(j, BK, s);
            }
        }
        lds_barrier();
        for (int e = tid; e < count * Jc; e += nt) {
            uint32_t* p = s_src + e * c;  // (gl, t) -> row gl*J + t*c
            for (int a = 1; a < c; ++a) {
                const uint32_t v = p[a];
                int b = a - 1;
                while (b >= 0 && (p[b] & ~kNeg) > (v & ~kNeg)) {
                    p[b + 1] = p[b];
                    --b;
                }
                p[b + 1] = v;
            }
        }
    } else {
        for (int e = tid; e < total; e += nt) {
            const int j = gi[e];
            const int s = gs[e];
            s_src[e] = (j >= 0 && j < J && (s == 1 || s == -1)) ? make_entry(j, BK, s) : kAbsent;
        }
    }
    lds_barrier();
}

// W_c fragments are read from global memory in a coalesced pattern (lane l
// reads 16 bytes at row l/4, k-chunk l%4, so each group of 4 lanes reads 64
// contiguous bytes of one row) and then moved into the MFMA operand pattern
// (lane l holds row l%16, k-chunk l/16) with a fixed cross-lane permutation.
// Read straight in the operand pattern, consecutive lanes would touch
// different rows and every lane quad different cache lines.
__device__ __forceinline__ int coalesced_src_lane_bytes(int lane) {
    return ((lane & 15) * 4 + (lane >> 4)) * 4;
}

__device__ __forceinline__ uint4 to_operand_layout(const uint4& v, int src_bytes) {
    uint4 r;
    r.x = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src_bytes, static_cast<int>(v.x)));
    r.y = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src_bytes, static_cast<int>(v.y)));
    r.z = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src_bytes, static_cast<int>(v.z)));
    r.w = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src_bytes, static_cast<int>(v.w)));
    return r;
}

// --------------------------------- weight operands from whole-line loads
// The 16x16x32 MFMA operand of a 16-row weight block wants, in lane l, row
// l%16 at 8 consecutive columns 8*(l/16) of a 32-wide k-step: 16 rows x 64
// bytes per load, half of every 128-byte line.  Two consecutive k-steps (64
// bf16 columns, one line per row) are loaded instead as two loads of 8 rows x
// 128 bytes (whole lines): lane l reads row l%8 (plus 8 for the second load)
// at the 16-byte piece (l/16) + 4*((l/8)%2) of the pair's 128 bytes, and
// pair_operands turns the two loads into the two steps' operands.

// Byte offset of lane l's piece in the first load of a pair, rows Kc
// elements apart (add 8 rows for the second load, and the pair's columns).
__device__ __forceinline__ uint32_t pair_load_offset(int lane, int Kc) {
    return static_cast<uint32_t>(((lane & 7) * Kc + ((lane >> 4) + 4 * ((lane >> 3) & 1)) * 8) * 2);
}

// All ones in lanes with l%16 < 8.
__device__ __forceinline__ uint32_t pair_lane_mask(int lane) { return (lane & 8) ? 0u : 0xFFFFFFFFu; }

// Lane l of a 16-lane row takes the value of lane (l + 8) % 16 (DPP
// row_ror:8, a VALU operand modifier; no LDS traffic).  Every lane is a
// valid source, so no old value is kept.
__device__ __forceinline__ uint32_t rot8(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x128, 0xF, 0xF, true));
}

// (p & m) | (q & ~m) in one v_bitop3_b32 (truth table 0xCA over the operands
// m, p, q: bit m ? p : q).  The operand choices below are bit selects on a
// lane mask, not conditionals: a conditional may become a branch, and a
// rotation issued under it would read lanes that the branch switched off.
__device__ __forceinline__ uint32_t bit_select(uint32_t m, uint32_t p, uint32_t q) {
    return __builtin_amdgcn_bitop3_b32(m, p, q, 0xCA);
}

// The two MFMA weight operands of a pair of k-steps from the pair's two loads
// a (rows 0..7 of the row block) and b (rows 8..15); lane l of a load holds
// row l%8 at the 16-byte piece (l/16) + 4*((l/8)%2) of the pair's 128 bytes.
// Operand lane l wants row l%16 at piece l/16 (first step) or 4 + l/16
// (second).  With lo8 all ones in lanes l%16 < 8: the first step's operand
// is a in those lanes and b rotated by 8 in the others; the second step's is
// a rotated by 8 in those lanes and b in the others.  One rotation of b
// merged with a serves both.
__device__ __forceinline__ void pair_operands(const uint4& a, const uint4& b, uint32_t lo8, uint4& t0, uint4& t1) {
    const uint4 e = {rot8(bit_select(lo8, b.x, a.x)), rot8(bit_select(lo8, b.y, a.y)),
                     rot8(bit_select(lo8, b.z, a.z)), rot8(bit_select(lo8, b.w, a.w))};
    t0.x = bit_select(lo8, a.x, e.x);
    t0.y = bit_select(lo8, a.y, e.y);
    t0.z = bit_select(lo8, a.z, e.z);
    t0.w = bit_select(lo8, a.w, e.w);
    t1.x = bit_select(lo8, e.x, b.x);
    t1.y = bit_select(lo8, e.y, b.y);
    t1.z = bit_select(lo8, e.z, b.z);
    t1.w = bit_select(lo8, e.w, b.w);
}

// Blocks are dealt to the 8 XCDs round-robin (block b runs on XCD b % 8).
// Renumber so that each XCD works through one contiguous range of tiles and
// tiles sharing an input row band stay in one L2.  A bijection on [0, n).
__device__ __forceinline__ int xcd_tile(int b, int n) {
    const int per = n / 8;
    if (b >= per * 8) return b;
    return (b % 8) * per + b / 8;
}

// ------------------------------------------------------------ fp8 weights
// Eight OCP E4M3 values (bytes, element 0 lowest) to eight bf16 values in the
// uint4 layout of a bf16 row: every E4M3 value (subnormals included) is a
// bf16 value, so the conversion (v_cvt_scalef32_pk_bf16_fp8, scale 1) is exact.
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint2 r) {
    uint4 o;
    o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.x, 1.0f, false));
    o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.x, 1.0f, true));
    o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.y, 1.0f, false));
    o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.y, 1.0f, true));
    return o;
}

// Raw storage of 8 consecutive weights: 16 bytes of bf16, or 8 bytes of E4M3.
template <bool W8>
struct WRaw {
    uint4 v;
    __device__ __forceinline__ void load(const uint16_t* w, size_t elem) {
        v = *reinterpret_cast<const uint4*>(w + elem);
    }
    __device__ __forceinline__ uint4 bf16() const { return v; }
};
template <>
struct WRaw<true> {
    uint2 v;
    __device__ __forceinline__ void load(const uint16_t* w, size_t elem) {
        v = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(w) + elem);
    }
    __device__ __forceinline__ uint4 bf16() const { return fp8x8_to_bf16x8(v); }
};

// ------------------------------------------------- transposing LDS operand read
// ds_read_b64_tr_b16 (gfx950), measured lane layout: inside each group of 16
// lanes, lane l receives element (l % 4) of the 8-byte piece addressed by lane
// 4i + l/4, for i = 0..3.  So from a row-major LDS tile S (pitch in elements)
// whose rows run along the MFMA reduction index, the 16x16x32 operand of
// column block n0 and reduction rows k0..k0+31 -- lane l holds
// S[k0 + 8*(l/16) + e][n0 + l%16], e = 0..7 -- comes from two such reads:
// lane l addresses row k0 + 8*(l/16) + 4h + (l%16)/4, column n0 + 4*(l%4), h = 0, 1.
// Rows must start 8-byte aligned (pitch % 4 == 0, n0 % 4 == 0).
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 lds_operand_tr(const uint16_t* S, int pitch, int k0, int n0, int lane) {
    const int q = lane >> 4;
    const int s = lane & 15;
    const uint16_t* p = S + (k0 + 8 * q + (s >> 2)) * pitch + n0 + 4 * (s & 3);
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * pitch));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// Output activation applied in the epilogues, on the float32 accumulator
// before the output rounding: kActNone, or kActGelu for GELU in its erf
// form, v * Phi(v) = 0.5 * v * (1 + erf(v / sqrt(2))).  Phi comes from the
// rational approximation of erf in Abramowitz & Stegun, Handbook of
// Mathematical Functions, formula 7.1.26 (absolute error at most 1.5e-7):
// with x = |v| / sqrt(2) and t = 1 / (1 + p x), 1 - erf(x) = (a1 t + a2 t^2 +
// a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2).  For v < 0, Phi(v) = (1 - erf(x)) / 2
// is formed directly, so the negative tail has no 1 + erf cancellation.  The
// epilogue runs while the matrix cores idle; this form costs a reciprocal, an
// exponential and a few fused multiply-adds.
__device__ __forceinline__ float apply_act(float v, int act) {
    if (act != kActGelu) return v;
    const float x = fabsf(v) * 0.70710678118654752440f;
    const float t = __frcp_rn(fmaf(0.3275911f, x, 1.0f));
    const float p = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f), -0.284496736f),
                             0.254829592f);
    const float q = 0.5f * p * __expf(-x * x);  // (1 - erf(x)) / 2 = Phi(-|v|)
    return v * (v >= 0.0f ? 1.0f - q : q);
}

}  // namespace dev
}  // namespace ss1
