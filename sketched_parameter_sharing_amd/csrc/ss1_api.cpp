// The C ABI of the SS1 forward library: argument checks, then kernel choice
// and launch.  Every check runs on the host before any HIP call, so a call
// that fails a check has enqueued nothing.
#include <stdint.h>

#include "ss1_group.h"
#include "ss1_internal.h"

using ss1::Dims;
using ss1::ForwardArgs;
using ss1::PlanForm;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_dtype(int32_t t) { return t == SS1_F32 || t == SS1_BF16; }

// Shapes, dtypes and alignment of one forward call.  Fills `a` on success.
ss1_status check_forward(const ss1_tensor* x, const ss1_tensor* W_c, const int32_t* plan_i,
                         const int8_t* plan_s, int32_t c, int32_t BK, int32_t BN,
                         const ss1_tensor* y, PlanForm form, void* stream, ForwardArgs* a) {
    if (!x || !W_c || !y) return SS1_ERR_NULL;
    if (x->reserved != 0 || W_c->reserved != 0 || y->reserved != 0) return SS1_ERR_SHAPE;
    if (!valid_dtype(x->dtype) || !valid_dtype(W_c->dtype) || !valid_dtype(y->dtype))
        return SS1_ERR_DTYPE;
    if (W_c->dtype != x->dtype || y->dtype != x->dtype) return SS1_ERR_DTYPE;
    const int64_t M = x->rows;
    const int64_t K = x->cols;
    const int64_t N = W_c->rows;
    Dims d;
    ss1_status st = ss1::check_chunking(K, N, c, BK, BN, &d);
    if (st != SS1_OK) return st;
    if (M < 0 || M > (int64_t(1) << 31) - 1) return SS1_ERR_SHAPE;
    if (K >= (int64_t(1) << 30) || N >= (int64_t(1) << 31)) return SS1_ERR_SHAPE;
    if (W_c->cols != d.Kc) return SS1_ERR_SHAPE;
    if (y->rows != M || y->cols != N) return SS1_ERR_SHAPE;
    if (x->dtype == SS1_BF16 ? (BK % 8 != 0) : (BK % 4 != 0)) return SS1_ERR_SHAPE;
    // element counts of each matrix must stay below 2^62 bytes of addressing
    if (M > 0 && K > (int64_t(1) << 40) / M) return SS1_ERR_SHAPE;
    if (M > 0 && N > (int64_t(1) << 40) / M) return SS1_ERR_SHAPE;
    if (M > 0) {
        if (!x->data || !y->data) return SS1_ERR_NULL;
    }
    if (!W_c->data || !plan_i || !plan_s) return SS1_ERR_NULL;
    if (!aligned(x->data, 16) || !aligned(W_c->data, 16) || !aligned(y->data, 16))
        return SS1_ERR_ALIGN;
    if (!aligned(plan_i, 4)) return SS1_ERR_ALIGN;
    a->x = x->data;
    a->w = W_c->data;
    a->y = y->data;
    a->plan_i = plan_i;
    a->plan_s = plan_s;
    a->form = form;
    a->M = M;
    a->d = d;
    a->dtype = x->dtype;
    a->stream = stream;
    return SS1_OK;
}

// Estimated time in microseconds of the sketch kernels (band or fused) on a
// large-M bf16 call, fitted to MI355X measurements (inputs not in cache): about
// 0.17 ps per (group, token, input element) and 2x that with 128-neuron
// groups, or the compressed MFMA work at 0.6 PFLOP/s if larger.
double sketch_estimate_us(const ForwardArgs& a) {
    const double M = static_cast<double>(a.M), K = static_cast<double>(a.d.K);
    const double G = static_cast<double>(a.d.G), N = static_cast<double>(a.d.N);
    // c >= 8: the band and fused kernels run 4 waves per block, and the band
    // kernel measured about 1.65x this model on the GPT-2 L up-projection at
    // c = 8, BK = 32 (235 us)
    const double valu = G * M * K * 0.17e-6 * (a.d.BN >= 128 ? 2.0 : 1.0) * (a.d.c >= 8 ? 1.6 : 1.0);
    const double mfma = 2.0 * M * N * static_cast<double>(a.d.Kc) / 0.6e9;
    return valu > mfma ? valu : mfma;
}

// The kernel ss1_forward picks for a validated call: decode shapes go to the
// matrix-vector kernel (M <= 4), the decode kernel (up to 16 rows of x in
// LDS) or the small-M kernel; otherwise the fold kernel when its estimate is
// clearly (10%) below the sketch kernels', else the band kernel where a band
// of input rows fits in LDS, else the fused kernel.
int32_t auto_algo(const ForwardArgs& a) {
    if (ss1::gemv_supported(a)) return SS1_ALGO_GEMV;
    if (ss1::decode_supported(a)) return SS1_ALGO_DECODE;
    if (ss1::smallm_supported(a)) return SS1_ALGO_SMALLM;
    if (ss1::fold_supported(a) && ss1::fold_estimate_us(a) < 0.9 * sketch_estimate_us(a)) return SS1_ALGO_FOLD;
    if (ss1::band_supported(a, 48)) return SS1_ALGO_BAND;
    if (ss1::fused_supported(a)) return SS1_ALGO_FUSED;
    return SS1_ALGO_GENERIC;
}

// The kernel ss1_forward_fp8w runs (a.w_fp8 set), or -1 when none can: the
// same order as ss1_forward's -- matrix-vector or small-M for decode shapes,
// the fold where the time models put it clearly ahead, else the band kernel
// where a band of input rows fits in LDS (E4M3 weights with a fixed c), else
// the fused kernel.
int32_t fp8_algo(const ForwardArgs& a) {
    if (ss1::gemv_supported(a)) return SS1_ALGO_GEMV;
    if (ss1::smallm_supported(a)) return SS1_ALGO_SMALLM;
    if (!ss1::fused_supported(a)) return -1;
    if (ss1::fold_supported(a) && ss1::fold_estimate_us(a) < 0.9 * sketch_estimate_us(a)) return SS1_ALGO_FOLD;
    if (ss1::band_supported(a, 48)) return SS1_ALGO_BAND;
    return SS1_ALGO_FUSED;
}

// What ss1_forward_ws runs: the column-split decode (with its workspace)
// for 5 <= M <= 16 where the decode kernel cannot hold the 16 input rows in
// LDS, else ss1_forward's choice.  Measured with cold weights on the
// Llama-3-8B decode shapes at M = 16: down (K = 14336) 23.8-24.2 us on the
// small-M kernel, 19.2-19.4 split; gate/up (K = 4096) 16.6-17.3 on the decode
// kernel, 25.6 split.
int32_t ws_algo(const ForwardArgs& a, size_t* bytes) {
    *bytes = 0;
    if (a.M >= 5 && !ss1::decode_supported(a) && ss1::split_slices(a) > 0) {
        *bytes = ss1::split_workspace_bytes(a);
        return SS1_ALGO_SPLIT;
    }
    return auto_algo(a);
}

ss1_status launch_algo(const ForwardArgs& a, int32_t algo) {
    switch (algo) {
        case SS1_ALGO_SMALLM: return ss1::launch_smallm(a);
        case SS1_ALGO_GEMV: return ss1::launch_gemv(a);
        case SS1_ALGO_DECODE: return ss1::launch_decode(a);
        case SS1_ALGO_BAND: return ss1::launch_band(a);
        case SS1_ALGO_FUSED: return ss1::launch_fused(a);
        case SS1_ALGO_FOLD: return ss1::launch_fold(a);
        case SS1_ALGO_GROUP: return ss1::launch_group(a);
        default: return ss1::launch_generic(a);
    }
}

ss1_status run_forward(const ss1_tensor* x, const ss1_tensor* W_c, const int32_t* plan_i,
                       const int8_t* plan_s, int32_t c, int32_t BK, int32_t BN, ss1_tensor* y,
                       int32_t algo, PlanForm form, void* stream) {
    ForwardArgs a;
    ss1_status st = check_forward(x, W_c, plan_i, plan_s, c, BK, BN, y, form, stream, &a);
    if (st != SS1_OK) return st;
    switch (algo) {
        case SS1_ALGO_AUTO:
            if (a.M == 0) return SS1_OK;
            return launch_algo(a, auto_algo(a));
        case SS1_ALGO_FUSED:
            if (!ss1::fused_supported(a)) return SS1_ERR_ALGO;
            return a.M == 0 ? SS1_OK : ss1::launch_fused(a);
        case SS1_ALGO_SMALLM:
            if (!ss1::smallm_supported(a)) return SS1_ERR_ALGO;
            return a.M == 0 ? SS1_OK : ss1::launch_smallm(a);
        case SS1_ALGO_GEMV:
            if (!ss1::gemv_supported(a)) return SS1_ERR_ALGO;
            return a.M == 0 ? SS1_OK : ss1::launch_gemv(a);
        case SS1_ALGO_DECODE:
            if (!ss1::decode_supported(a)) return SS1_ERR_ALGO;
            return a.M == 0 ? SS1_OK : ss1::launch_decode(a);
        case SS1_ALGO_BAND:
            if (!ss1::band_supported(a, 32)) return SS1_ERR_ALGO;
            return a.M == 0 ? SS1_OK : ss1::launch_band(a);
        case SS1_ALGO_FOLD:
            if (!ss1::fold_supported(a)) return SS1_ERR_ALGO;
            return a.M == 0 ? SS1_OK : ss1::launch_fold(a);
        case SS1_ALGO_GROUP:
            if (!ss1::group_supported(a)) return SS1_ERR_ALGO;
            return a.M == 0 ? SS1_OK : ss1::launch_group(a);
        case SS1_ALGO_GENERIC:
            return a.M == 0 ? SS1_OK : ss1::launch_generic(a);
        default:
            return SS1_ERR_ALGO;
    }
}

}  // namespace

extern "C" const char* ss1_version(void) { return "0.1.0"; }

extern "C" const char* ss1_status_string(ss1_status s) {
    switch (s) {
        case SS1_OK: return "ok";
        case SS1_ERR_NULL: return "null pointer";
        case SS1_ERR_SHAPE: return "invalid or inconsistent shape";
        case SS1_ERR_DTYPE: return "invalid or mismatched dtype";
        case SS1_ERR_PLAN: return "invalid plan (range, sign or balance)";
        case SS1_ERR_ALIGN: return "misaligned pointer";
        case SS1_ERR_HIP: return "HIP launch or runtime error";
        case SS1_ERR_ALGO: return "requested kernel cannot run this call";
    }
    return "unknown status";
}

extern "C" ss1_status ss1_forward(const ss1_tensor* x, const ss1_tensor* W_c, const int32_t* hash,
                                  const int8_t* sign, int32_t c, int32_t BK, int32_t BN,
                                  ss1_tensor* y, void* stream) {
    return run_forward(x, W_c, hash, sign, c, BK, BN, y, SS1_ALGO_AUTO, PlanForm::Hash, stream);
}

extern "C" ss1_status ss1_forward_idx(const ss1_tensor* x, const ss1_tensor* W_c,
                                      const int32_t* idx, const int8_t* isign, int32_t c,
                                      int32_t BK, int32_t BN, ss1_tensor* y, void* stream) {
    return run_forward(x, W_c, idx, isign, c, BK, BN, y, SS1_ALGO_AUTO, PlanForm::Index, stream);
}

extern "C" ss1_status ss1_forward_algo(const ss1_tensor* x, const ss1_tensor* W_c,
                                       const int32_t* hash, const int8_t* sign, int32_t c,
                                       int32_t BK, int32_t BN, ss1_tensor* y, int32_t algo,
                                       void* stream) {
    return run_forward(x, W_c, hash, sign, c, BK, BN, y, algo, PlanForm::Hash, stream);
}

extern "C" ss1_status ss1_forward_idx_algo(const ss1_tensor* x, const ss1_tensor* W_c,
                                           const int32_t* idx, const int8_t* isign, int32_t c,
                                           int32_t BK, int32_t BN, ss1_tensor* y, int32_t algo,
                                           void* stream) {
    return run_forward(x, W_c, idx, isign, c, BK, BN, y, algo, PlanForm::Index, stream);
}

extern "C" ss1_status ss1_select_algo(const ss1_tensor* x, const ss1_tensor* W_c, int32_t c, int32_t BK,
                                      int32_t BN, int32_t* algo) {
    if (!x || !W_c || !algo) return SS1_ERR_NULL;
    // shape and dtype checks of ss1_forward on a stand-in output and plan
    ss1_tensor y{x->data, x->dtype, 0, x->rows, W_c->rows};
    static const int32_t plan_i = 0;
    static const int8_t plan_s = 0;
    ss1_tensor xs = *x, ws = *W_c;
    static char dummy[16] __attribute__((aligned(16)));
    if (!xs.data) xs.data = dummy;
    if (!ws.data) ws.data = dummy;
    y.data = xs.data;
    // E4M3 weights: the choice of ss1_forward_fp8w (bf16 x only)
    const bool fp8 = ws.dtype == SS1_FP8_E4M3;
    if (fp8) {
        if (xs.dtype != SS1_BF16) return SS1_ERR_DTYPE;
        ws.dtype = xs.dtype;
    }
    ForwardArgs a;
    ss1_status st = check_forward(&xs, &ws, &plan_i, &plan_s, c, BK, BN, &y, fp8 ? PlanForm::Hash : PlanForm::Index,
                                  nullptr, &a);
    if (st != SS1_OK) return st;
    if (fp8) {
        a.w_fp8 = true;
        const int32_t k = fp8_algo(a);
        if (k < 0) return SS1_ERR_SHAPE;
        *algo = k;
        return SS1_OK;
    }
    *algo = auto_algo(a);
    return SS1_OK;
}

extern "C" ss1_status ss1_forward_ws_query(const ss1_tensor* x, const ss1_tensor* W_c, int32_t c, int32_t BK,
                                           int32_t BN, size_t* bytes, int32_t* algo) {
    if (!x || !W_c || !bytes || !algo) return SS1_ERR_NULL;
    ss1_tensor y{x->data, x->dtype, 0, x->rows, W_c->rows};
    static const int32_t plan_i = 0;
    static const int8_t plan_s = 0;
    static char dummy[16] __attribute__((aligned(16)));
    ss1_tensor xs = *x, ws = *W_c;
    if (!xs.data) xs.data = dummy;
    if (!ws.data) ws.data = dummy;
    y.data = xs.data;
    ForwardArgs a;
    ss1_status st = check_forward(&xs, &ws, &plan_i, &plan_s, c, BK, BN, &y, PlanForm::Index, nullptr, &a);
    if (st != SS1_OK) return st;
    *algo = ws_algo(a, bytes);
    return SS1_OK;
}

extern "C" ss1_status ss1_forward_ws(const ss1_tensor* x, const ss1_tensor* W_c, const int32_t* hash,
                                     const int8_t* sign, int32_t c, int32_t BK, int32_t BN, ss1_tensor* y,
                                     void* workspace, size_t workspace_bytes, void* stream) {
    ForwardArgs a;
    ss1_status st = check_forward(x, W_c, hash, sign, c, BK, BN, y, PlanForm::Hash, stream, &a);
    if (st != SS1_OK) return st;
    size_t need = 0;
    const int32_t algo = ws_algo(a, &need);
    if (need > 0) {
        if (!workspace) return SS1_ERR_NULL;
        if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return SS1_ERR_ALIGN;
        if (workspace_bytes < need) return SS1_ERR_SHAPE;
    }
    if (a.M == 0) return SS1_OK;
    if (algo == SS1_ALGO_SPLIT) return ss1::launch_split(a, workspace);
    return launch_algo(a, algo);
}

extern "C" ss1_status ss1_sketch(const ss1_tensor* x, const int32_t* hash, const int8_t* sign,
                                 int32_t c, int32_t BK, int32_t BN, int64_t N, ss1_tensor* z,
                                 void* stream) {
    if (!x || !z) return SS1_ERR_NULL;
    if (x->reserved != 0 || z->reserved != 0) return SS1_ERR_SHAPE;
    if (!valid_dtype(x->dtype) || !valid_dtype(z->dtype)) return SS1_ERR_DTYPE;
    if (x->dtype == SS1_F32 && z->dtype != SS1_F32) return SS1_ERR_DTYPE;
    const int64_t M = x->rows;
    const int64_t K = x->cols;
    Dims d;
    ss1_status st = ss1::check_chunking(K, N, c, BK, BN, &d);
    if (st != SS1_OK) return st;
    if (M < 0 || M > (int64_t(1) << 31) - 1 || K >= (int64_t(1) << 30)) return SS1_ERR_SHAPE;
    if (x->dtype == SS1_BF16 ? (BK % 8 != 0) : (BK % 4 != 0)) return SS1_ERR_SHAPE;
    if (z->rows != d.G * M || z->cols != d.Kc) return SS1_ERR_SHAPE;
    if (d.G > 65535) return SS1_ERR_SHAPE;
    if (M > 0 && K > (int64_t(1) << 40) / M) return SS1_ERR_SHAPE;
    if (!hash || !sign) return SS1_ERR_NULL;
    if (M == 0) return SS1_OK;
    if (!x->data || !z->data) return SS1_ERR_NULL;
    if (!aligned(x->data, 16) || !aligned(z->data, 16)) return SS1_ERR_ALIGN;
    if (!aligned(hash, 4)) return SS1_ERR_ALIGN;
    return ss1::launch_sketch(x->data, x->dtype, hash, sign, M, d, z->data, z->dtype, stream);
}

extern "C" ss1_status ss1_project(const ss1_tensor* W, const int32_t* hash, const int8_t* sign, int32_t c,
                                  int32_t BK, int32_t BN, ss1_tensor* W_c, void* stream) {
    if (!W || !W_c) return SS1_ERR_NULL;
    if (W->reserved != 0 || W_c->reserved != 0) return SS1_ERR_SHAPE;
    if (!valid_dtype(W->dtype) || !valid_dtype(W_c->dtype)) return SS1_ERR_DTYPE;
    if (W_c->dtype != W->dtype) return SS1_ERR_DTYPE;
    const int64_t N = W->rows;
    const int64_t K = W->cols;
    Dims d;
    ss1_status st = ss1::check_chunking(K, N, c, BK, BN, &d);
    if (st != SS1_OK) return st;
    if (K >= (int64_t(1) << 30) || N >= (int64_t(1) << 31)) return SS1_ERR_SHAPE;
    if (N > (int64_t(1) << 40) / K) return SS1_ERR_SHAPE;
    if (W_c->rows != N || W_c->cols != d.Kc) return SS1_ERR_SHAPE;
    if (W->dtype == SS1_BF16 ? (BK % 8 != 0) : (BK % 4 != 0)) return SS1_ERR_SHAPE;
    if (d.G > 65535) return SS1_ERR_SHAPE;
    if (!W->data || !W_c->data || !hash || !sign) return SS1_ERR_NULL;
    if (!aligned(W->data, 16) || !aligned(W_c->data, 16)) return SS1_ERR_ALIGN;
    if (!aligned(hash, 4)) return SS1_ERR_ALIGN;
    return ss1::launch_project(W->data, W->dtype, hash, sign, d, W_c->data, stream);
}

namespace ss1 {

ss1_status mlp_forward_ws(const ss1_tensor* x, const ss1_layer* up, const ss1_layer* down, ss1_tensor* h,
                          ss1_tensor* y, void* stream) {
    if (!x || !up || !down || !h || !y) return SS1_ERR_NULL;
    if (up->reserved != 0 || down->reserved != 0 || h->reserved != 0) return SS1_ERR_SHAPE;
    const int64_t M = x->rows;
    const int64_t R = h->rows;
    if (M < 0) return SS1_ERR_SHAPE;
    if (M > 0 && R < 1) return SS1_ERR_SHAPE;
    const int64_t RC = M > 0 ? (R < M ? R : M) : 0;  // rows per chunk
    // whole-call checks: the up layer maps x to h's columns, the down layer
    // h's columns to y, on descriptors of the first chunk's shape
    ss1_tensor xc = *x, hc = *h, yc = *y;
    xc.rows = RC;
    hc.rows = RC;
    yc.rows = RC;
    ForwardArgs au, ad;
    ss1_status st = check_forward(&xc, &up->W_c, up->hash, up->sign, up->c, up->BK, up->BN, &hc, PlanForm::Hash,
                                  stream, &au);
    if (st != SS1_OK) return st;
    st = check_forward(&hc, &down->W_c, down->hash, down->sign, down->c, down->BK, down->BN, &yc, PlanForm::Hash,
                       stream, &ad);
    if (st != SS1_OK) return st;
    // the full-size x and y, and the workspace's own shape
    if (y->rows != M || y->cols != down->W_c.rows) return SS1_ERR_SHAPE;
    if (h->cols != up->W_c.rows || h->dtype != x->dtype) return SS1_ERR_SHAPE;
    if (M > 0 && x->cols > (int64_t(1) << 40) / M) return SS1_ERR_SHAPE;
    if (M > 0 && y->cols > (int64_t(1) << 40) / M) return SS1_ERR_SHAPE;
    if (M > (int64_t(1) << 31) - 1) return SS1_ERR_SHAPE;
    if (M == 0) return SS1_OK;
    const size_t e = x->dtype == SS1_BF16 ? 2 : 4;
    au.act = ss1::kActGelu;
    for (int64_t r0 = 0; r0 < M; r0 += RC) {
        const int64_t rows = (M - r0 < RC) ? (M - r0) : RC;
        au.x = static_cast<const char*>(x->data) + static_cast<size_t>(r0) * x->cols * e;
        au.M = rows;
        ad.y = static_cast<char*>(y->data) + static_cast<size_t>(r0) * y->cols * e;
        ad.M = rows;
        st = launch_algo(au, auto_algo(au));
        if (st != SS1_OK) return st;
        st = launch_algo(ad, auto_algo(ad));
        if (st != SS1_OK) return st;
    }
    return SS1_OK;
}

}  // namespace ss1

extern "C" ss1_status ss1_mlp_forward(const ss1_tensor* x, const ss1_layer* up, const ss1_layer* down,
                                      ss1_tensor* h, ss1_tensor* y, void* stream) {
    return ss1::mlp_forward_ws(x, up, down, h, y, stream);
}

extern "C" ss1_status ss1_quantize_fp8(const ss1_tensor* W_c, ss1_tensor* Q, float* scale, void* stream) {
    if (!W_c || !Q) return SS1_ERR_NULL;
    if (W_c->reserved != 0 || Q->reserved != 0) return SS1_ERR_SHAPE;
    if (!valid_dtype(W_c->dtype) || Q->dtype != SS1_FP8_E4M3) return SS1_ERR_DTYPE;
    const int64_t N = W_c->rows;
    const int64_t Kc = W_c->cols;
    if (N < 0 || Kc < 2 || Kc % 2 != 0 || Kc >= (int64_t(1) << 30) || N >= (int64_t(1) << 31)) return SS1_ERR_SHAPE;
    if (Q->rows != N || Q->cols != Kc) return SS1_ERR_SHAPE;
    if (N > (int64_t(1) << 40) / Kc) return SS1_ERR_SHAPE;
    if (N == 0) return SS1_OK;
    if (!W_c->data || !Q->data || !scale) return SS1_ERR_NULL;
    if (!aligned(W_c->data, 16) || !aligned(Q->data, 16) || !aligned(scale, 4)) return SS1_ERR_ALIGN;
    return ss1::launch_quantize_fp8(W_c->data, W_c->dtype, N, Kc, Q->data, scale, stream);
}

extern "C" ss1_status ss1_forward_fp8w(const ss1_tensor* x, const ss1_tensor* Q, const float* scale,
                                       const int32_t* hash, const int8_t* sign, int32_t c, int32_t BK,
                                       int32_t BN, ss1_tensor* y, void* stream) {
    if (!x || !Q || !y) return SS1_ERR_NULL;
    if (Q->dtype != SS1_FP8_E4M3) return SS1_ERR_DTYPE;
    if (x->dtype != SS1_BF16) return SS1_ERR_DTYPE;
    // the forward's own checks, on a descriptor of W_c's shape in x's dtype
    ss1_tensor wq = *Q;
    wq.dtype = x->dtype;
    ForwardArgs a;
    ss1_status st = check_forward(x, &wq, hash, sign, c, BK, BN, y, PlanForm::Hash, stream, &a);
    if (st != SS1_OK) return st;
    if (!scale) return SS1_ERR_NULL;
    if (!aligned(scale, 4)) return SS1_ERR_ALIGN;
    a.w_fp8 = true;
    a.wscale = scale;
    const int32_t algo = fp8_algo(a);
    if (algo < 0) return SS1_ERR_SHAPE;
    if (a.M == 0) return SS1_OK;
    if (algo == SS1_ALGO_GEMV) return ss1::launch_gemv(a);
    if (algo == SS1_ALGO_SMALLM) return ss1::launch_smallm(a);
    if (algo == SS1_ALGO_FOLD) return ss1::launch_fold(a);
    if (algo == SS1_ALGO_BAND) return ss1::launch_band(a);
    return ss1::launch_fused(a);
}

extern "C" ss1_status ss1_forward_fp8(const ss1_tensor* xq, const float* xscale, const ss1_tensor* Wq,
                                      const float* wscale, const int32_t* hash, const int8_t* sign, int32_t c,
                                      int32_t BK, int32_t BN, ss1_tensor* y, void* stream) {
    if (!xq || !Wq || !y) return SS1_ERR_NULL;
    if (xq->dtype != SS1_FP8_E4M3 || Wq->dtype != SS1_FP8_E4M3 || y->dtype != SS1_BF16) return SS1_ERR_DTYPE;
    // the forward's own checks, on descriptors of the same shapes in bf16
    ss1_tensor xb = *xq, wb = *Wq;
    xb.dtype = SS1_BF16;
    wb.dtype = SS1_BF16;
    ForwardArgs a;
    ss1_status st = check_forward(&xb, &wb, hash, sign, c, BK, BN, y, PlanForm::Hash, stream, &a);
    if (st != SS1_OK) return st;
    if (!wscale || (a.M > 0 && !xscale)) return SS1_ERR_NULL;
    if (!aligned(wscale, 4) || !aligned(xscale, 4)) return SS1_ERR_ALIGN;
    if (!ss1::fold8_supported(a.M, a.d)) return SS1_ERR_SHAPE;
    if (a.M == 0) return SS1_OK;
    return ss1::launch_fold8(xq->data, xscale, Wq->data, wscale, hash, sign, y->data, a.M, a.d, ss1::kActNone,
                             stream);
}

extern "C" ss1_status ss1_backward_select_algo(const ss1_tensor* x, const ss1_tensor* W_c, int32_t c,
                                               int32_t BK, int32_t BN, int32_t* dx_algo, int32_t* dw_algo) {
    if (!x || !W_c || !dx_algo || !dw_algo) return SS1_ERR_NULL;
    // the shape and dtype checks of ss1_backward on stand-in buffers
    static char dummy[16] __attribute__((aligned(16)));
    static const int32_t plan_i = 0;
    static const int8_t plan_s = 0;
    ss1_tensor xs = *x, ws = *W_c;
    if (!xs.data) xs.data = dummy;
    if (!ws.data) ws.data = dummy;
    ss1_tensor dy{xs.data, xs.dtype, 0, xs.rows, ws.rows};
    ForwardArgs a;
    ss1_status st = check_forward(&xs, &ws, &plan_i, &plan_s, c, BK, BN, &dy, PlanForm::Hash, nullptr, &a);
    if (st != SS1_OK) return st;
    if (xs.dtype != SS1_BF16) return SS1_ERR_DTYPE;
    if (BK % 32 != 0 || BN % 32 != 0) return SS1_ERR_SHAPE;
    if (a.d.G > 8192) return SS1_ERR_SHAPE;
    // the choice ss1_backward makes: dW_c on the fold kernel (no sketch) when
    // its shape rules hold, else on the sketch kernel; dx on the fold kernel
    // when its rules hold, else on the tiled dx kernels (no sketch either way)
    *dw_algo = ss1::dw_fold_supported(a.M, a.d) ? SS1_ALGO_FOLD : SS1_ALGO_FUSED;
    *dx_algo = ss1::dx_fold_supported(a.M, a.d) ? SS1_ALGO_FOLD : SS1_ALGO_GENERIC;
    return SS1_OK;
}

extern "C" ss1_status ss1_backward(const ss1_tensor* x, const ss1_tensor* W_c, const int32_t* hash,
                                   const int8_t* sign, int32_t c, int32_t BK, int32_t BN, const ss1_tensor* dy,
                                   ss1_tensor* dx, ss1_tensor* dW_c, void* stream) {
    if (!x || !W_c || !dy) return SS1_ERR_NULL;
    if (!dx && !dW_c) return SS1_OK;
    // the forward's checks of x, W_c and the plan, with dy in y's place
    ForwardArgs a;
    ss1_status st = check_forward(x, W_c, hash, sign, c, BK, BN, dy, PlanForm::Hash, stream, &a);
    if (st != SS1_OK) return st;
    if (x->dtype != SS1_BF16) return SS1_ERR_DTYPE;
    if (BK % 32 != 0 || BN % 32 != 0) return SS1_ERR_SHAPE;
    if (a.d.G > 8192 || a.M > (int64_t(1) << 31) - 1) return SS1_ERR_SHAPE;
    if (dx) {
        if (dx->reserved != 0) return SS1_ERR_SHAPE;
        if (dx->dtype != SS1_BF16) return SS1_ERR_DTYPE;
        if (dx->rows != a.M || dx->cols != a.d.K) return SS1_ERR_SHAPE;
        if (a.M > 0 && !dx->data) return SS1_ERR_NULL;
        if (!aligned(dx->data, 16)) return SS1_ERR_ALIGN;
    }
    if (dW_c) {
        if (dW_c->reserved != 0) return SS1_ERR_SHAPE;
        if (dW_c->dtype != SS1_BF16) return SS1_ERR_DTYPE;
        if (dW_c->rows != a.d.N || dW_c->cols != a.d.Kc) return SS1_ERR_SHAPE;
        if (!dW_c->data) return SS1_ERR_NULL;
        if (!aligned(dW_c->data, 16)) return SS1_ERR_ALIGN;
    }
    return ss1::launch_backward(x->data, W_c->data, hash, sign, dy->data, dx ? dx->data : nullptr,
                                dW_c ? dW_c->data : nullptr, a.M, a.d, stream);
}
