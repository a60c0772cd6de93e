// Internal declarations shared by the host ABI layer and the kernel launchers.
#pragma once

#include <stdint.h>

#include "../../include/ss1.h"

namespace ss1 {

struct Dims {
    int64_t K, N;
    int32_t c, BK, BN;
    int64_t J, Jc, Kc, G;
};

// Checks the chunking (K % BK, (K/BK) % c, N % BN, ranges) and fills `d`.
ss1_status check_chunking(int64_t K, int64_t N, int32_t c, int32_t BK, int32_t BN, Dims* d);

// How the device reads the plan: the forward hash/sign [G][J], or the inverse
// index idx/isign [G][Jc][c].
enum class PlanForm { Hash, Index };

struct ForwardArgs {
    const void* x;
    const void* w;
    void* y;
    const int32_t* plan_i;
    const int8_t* plan_s;
    PlanForm form;
    int64_t M;
    Dims d;
    int32_t dtype;  // ss1_dtype
    void* stream;
    int32_t act = 0;  // epilogue activation: kActNone or kActGelu (erf form)
    // fp8 weights: w holds OCP E4M3 codes and wscale one float per row
    bool w_fp8 = false;
    const float* wscale = nullptr;
};

// Epilogue activation codes (ForwardArgs::act; applied by dev::apply_act).
constexpr int32_t kActNone = 0;
constexpr int32_t kActGelu = 1;

// Which kernels can run a call (host-side checks only).
bool fused_supported(const ForwardArgs& a);
bool smallm_supported(const ForwardArgs& a);
// Matrix-vector kernel (ss1_gemv.hip): bf16, M <= 4, BN % 16 == 0, 512 to
// 65536 compressed columns (fewer for M > 1) and J within twice the block.
bool gemv_supported(const ForwardArgs& a);
// Decode kernel (ss1_decode.hip): bf16, M <= 16, K % 512 == 0 with 16 input
// rows of K bf16 in LDS, BN of 32 or 64, BK % 32 == 0, J <= 2048.
bool decode_supported(const ForwardArgs& a);
// Column-split decode (ss1_decode.hip): slices per group (0 when it does not
// apply), the float32 workspace it needs (Q * M * N floats), and the launch
// (split kernel, then the in-order sum of the slices into y).
int split_slices(const ForwardArgs& a);
size_t split_workspace_bytes(const ForwardArgs& a);
ss1_status launch_split(const ForwardArgs& a, void* workspace);
// Band kernel: the layer's rows are short enough for a band of at least
// min_rows input rows to sit in LDS.
bool band_supported(const ForwardArgs& a, int min_rows);
// Fold kernel (ss1_fold.hip): bf16, BK % 32 == 0, a 128- or 256-neuron tile of
// whole groups that divides N.
bool fold_supported(const ForwardArgs& a);
// Estimated fold-kernel time in microseconds (huge when it cannot run).
double fold_estimate_us(const ForwardArgs& a);
// Backward dx as the fold contraction (ss1_fold.hip): bf16, hash plan,
// N % 64 == 0, K % 256 == 0, BK % 64 == 0 and the plan table in LDS.
bool dx_fold_supported(int64_t M, const Dims& d);
ss1_status launch_dx_fold(const void* dy, const void* W_c, const int32_t* hash, const int8_t* sign, void* dx,
                          int64_t M, const Dims& d, void* stream);
// Backward dW_c as the fold contraction over (token, source) (ss1_fold.hip):
// bf16, hash plan, BN % 64 == 0, BK % 64 == 0, c in {1, 2, 4}, Kc % 128 == 0.
bool dw_fold_supported(int64_t M, const Dims& d);
// Both gradients in one fold launch (dW_c tiles and dx tiles share the grid)
// where both fold kernels apply and their configurations pair up.
bool bwd_fold_supported(int64_t M, const Dims& d);
ss1_status launch_bwd_fold(const void* x, const void* W_c, const int32_t* hash, const int8_t* sign, const void* dy,
                           void* dx, void* dW, int64_t M, const Dims& d, void* stream);
ss1_status launch_dw_fold(const void* x, const void* dy, const int32_t* hash, const int8_t* sign, void* dW,
                          int64_t M, const Dims& d, void* stream);

// The MLP pair (ss1_mlp_forward's checks and chunked launches) with h as the
// per-chunk workspace; every check runs before any HIP call.
ss1_status mlp_forward_ws(const ss1_tensor* x, const ss1_layer* up, const ss1_layer* down, ss1_tensor* h,
                          ss1_tensor* y, void* stream);

// fp8 fold (ss1_fold.hip): x and W_c both as E4M3 codes with float32 row
// scales, bf16 y; hash plan; N % 256 == 0, 256 % BN == 0, BK % 64 == 0,
// K % 128 == 0.
bool fold8_supported(int64_t M, const Dims& d);
ss1_status launch_fold8(const void* xq, const float* xs, const void* wq, const float* ws, const int32_t* hash,
                        const int8_t* sign, void* y, int64_t M, const Dims& d, int32_t act, void* stream);

// Kernel launchers (ss1_kernels.hip).  Return SS1_OK or SS1_ERR_HIP.
ss1_status launch_fused(const ForwardArgs& a);
ss1_status launch_smallm(const ForwardArgs& a);
ss1_status launch_gemv(const ForwardArgs& a);
ss1_status launch_decode(const ForwardArgs& a);
ss1_status launch_band(const ForwardArgs& a);
ss1_status launch_generic(const ForwardArgs& a);
ss1_status launch_fold(const ForwardArgs& a);
ss1_status launch_sketch(const void* x, int32_t x_dtype, const int32_t* plan_i, const int8_t* plan_s,
                         int64_t M, const Dims& d, void* z, int32_t z_dtype, void* stream);
// Backward: dW_c (when dW is not null) and dx (when dx is not null), bf16,
// plan in the forward hash form (ss1_backward.hip).
ss1_status launch_backward(const void* x, const void* W_c, const int32_t* hash, const int8_t* sign, const void* dy,
                           void* dx, void* dW, int64_t M, const Dims& d, void* stream);
// Per-row E4M3 quantization of a compressed weight (ss1_quant.hip).
ss1_status launch_quantize_fp8(const void* W, int32_t dtype, int64_t N, int64_t Kc, void* Q, float* scale,
                               void* stream);
// Projection of a dense [N][K] weight onto the sharing pattern (ss1_project.hip).
ss1_status launch_project(const void* W, int32_t dtype, const int32_t* hash, const int8_t* sign, const Dims& d,
                          void* Wc, void* stream);

}  // namespace ss1
