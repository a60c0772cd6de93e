/*
 * ss1.h -- C ABI of the SS1 (Sketch Structured Transform) forward library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (source: "SS1: Accelerating Inference with Fast and Expressive
 * Sketch Structured Transform", summary page, section "Approach"; and the SS1
 * author abstract): a linear layer whose neurons share parameters randomly but
 * only inside their own weight vector, through hash functions coalesced along
 * K and along N.  The layer first sketches its input down by the compression
 * factor c using additions and subtractions only, then multiplies the sketch
 * by the compressed weight W_c, so it does c times fewer FLOPs than the dense
 * layer it replaces.
 *
 * Concretely (readings of the page's wording, fixed here):
 *   J  = K / BK input chunks of BK consecutive inputs, Jc = J / c, Kc = K / c,
 *   G  = N / BN neuron groups of BN consecutive neurons (n belongs to n / BN).
 *   Plan of group g: hash[g][j] in [0, Jc) and sign[g][j] in {-1, +1}; it is
 *   balanced: every compressed chunk t receives exactly c input chunks.
 *   Sketch:  z_g[m][t*BK + u] = sum over j with hash[g][j] == t of
 *                               sign[g][j] * x[m][j*BK + u]
 *   Output:  y[m][n] = sum over k' < Kc of z_{n/BN}[m][k'] * W_c[n][k']
 *
 * Layouts: every matrix is dense row-major with rows packed (row stride =
 * cols).  x is [M][K], W_c is [N][Kc] (one row per neuron, like a dense
 * layer's [out][in] weight), y is [M][N].  hash/sign are [G][J]; the inverse
 * index idx/isign is [G][Jc][c].
 *
 * Precision: float32 layers compute the sketch and the contraction in float32
 * (fused multiply-add, no reduced-precision matrix format).  bf16 layers sum
 * each sketch value in float32 over its sources in ascending chunk order,
 * round it to bf16 (nearest, ties to even), contract on bf16 matrix cores with
 * float32 accumulation, and round y to bf16 (nearest, ties to even).
 *
 * Ownership and threading: the caller owns every buffer.  The device entry
 * points do not allocate, free or cache anything and keep no global state;
 * they enqueue work on the caller's HIP stream and return without waiting.
 * They are safe to call from several threads at once.
 *
 * Errors: every call returns an ss1_status.  All argument checks (null
 * pointers, shapes, dtypes, alignment) happen on the host before any HIP call,
 * so a failing check enqueues nothing.  A failed launch returns SS1_ERR_HIP;
 * faults during execution surface at the caller's next synchronisation.
 */
#ifndef SS1_H
#define SS1_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SS1_OK = 0,
    SS1_ERR_NULL = 1,      /* a required pointer is NULL                          */
    SS1_ERR_SHAPE = 2,     /* sizes inconsistent, non-dividing or out of range   */
    SS1_ERR_DTYPE = 3,     /* unknown dtype, or x / W_c / y dtypes differ         */
    SS1_ERR_PLAN = 4,      /* host plan arrays fail validation (range, sign, balance) */
    SS1_ERR_ALIGN = 5,     /* a device pointer is not aligned as documented       */
    SS1_ERR_HIP = 6,       /* a HIP launch or runtime call failed                 */
    SS1_ERR_ALGO = 7       /* the requested kernel cannot run this shape          */
} ss1_status;

/* Element types.  SS1_FP8_E4M3 (OCP 8-bit float E4M3, one byte per element)
   is only for quantized compressed weights (ss1_quantize_fp8,
   ss1_forward_fp8w). */
typedef enum { SS1_F32 = 0, SS1_BF16 = 1, SS1_FP8_E4M3 = 2 } ss1_dtype;

/* Kernel choice for ss1_forward_algo / ss1_forward_idx_algo. */
typedef enum {
    SS1_ALGO_AUTO = 0,     /* what ss1_forward picks                                  */
    SS1_ALGO_FUSED = 1,    /* bf16: sketch tile built in LDS, then MFMA (M of any size) */
    SS1_ALGO_SMALLM = 2,   /* bf16: decode shapes, M <= 16, W_c streamed once          */
    SS1_ALGO_GENERIC = 3,  /* any dtype and chunking: LDS-tiled FMA kernel             */
    SS1_ALGO_BAND = 4,     /* bf16, short rows: a band of input rows held in LDS        */
    SS1_ALGO_FOLD = 5,     /* bf16: W_c expanded on chip, one dense-shaped MFMA GEMM    */
    SS1_ALGO_GEMV = 6,     /* bf16: M <= 4, matrix-vector kernel, W_c streamed once     */
    SS1_ALGO_DECODE = 7,   /* bf16: M <= 16 with 16 input rows in LDS, one group per
                              block, every weight load in flight, MFMA               */
    SS1_ALGO_SPLIT = 8,    /* bf16: M <= 16, each group's compressed columns split over
                              blocks, partial sums in a caller workspace (ss1_forward_ws
                              only)                                                  */
    SS1_ALGO_GROUP = 9     /* bf16, c in {2, 4, 8}, BK % 64 == 0, BN 64 or 128: one
                              neuron group per block, the sketch formed on the matrix
                              cores, only the compressed contraction                 */
} ss1_algo;

/* A dense row-major matrix in device memory (rows packed). */
typedef struct {
    void* data;
    int32_t dtype;         /* ss1_dtype */
    int32_t reserved;      /* must be 0 */
    int64_t rows;
    int64_t cols;
} ss1_tensor;

/* One SS1 layer for the calls that take several: its compressed weight and
   its plan.  All pointers are the caller's; the library keeps none. */
typedef struct {
    ss1_tensor W_c;        /* [N][K/c] row-major, DEVICE */
    const int32_t* hash;   /* DEVICE [G][J] as written by ss1_plan */
    const int8_t* sign;    /* DEVICE [G][J] */
    int32_t c;
    int32_t BK;
    int32_t BN;
    int32_t reserved;      /* must be 0 */
} ss1_layer;

/* Largest number of input chunks J = K/BK per group the device kernels take
   (their plan is staged in LDS). */
#define SS1_MAX_CHUNKS 4096
/* Largest compression factor. */
#define SS1_MAX_C 64

/* Library version, "major.minor.patch". */
const char* ss1_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* ss1_status_string(ss1_status s);

/*
 * ss1_plan -- HOST.  Seeded balanced chunk hash and +-1 signs for every group
 * (the random, within-neuron, K- and N-coalesced parameter sharing of the SS1
 * summary page, "Approach"; the generator itself is this library's choice):
 *   SplitMix64 (Steele, Lea, Flood 2014) seeded with `seed`; for g = 0..G-1 in
 *   order: Fisher-Yates shuffle of [0, J) (i from J-1 down to 1, swap i with
 *   next() % (i+1)); the chunk at shuffled position p gets hash p / c; then one
 *   draw per chunk j = 0..J-1, sign = -1 when its top bit is set, else +1.
 * Outputs: caller-owned host arrays hash[G*J] (int32) and sign[G*J] (int8),
 * row-major [G][J].  Deterministic in (seed, K, N, c, BK, BN).
 * Errors: SS1_ERR_NULL, SS1_ERR_SHAPE (K % BK, (K/BK) % c, N % BN, non-positive
 * sizes, c > SS1_MAX_C, J > SS1_MAX_CHUNKS).
 */
ss1_status ss1_plan(uint64_t seed, int64_t K, int64_t N, int32_t c, int32_t BK, int32_t BN,
                    int32_t* hash, int8_t* sign);

/*
 * ss1_plan_index -- HOST.  Validates a plan (0 <= hash < Jc, sign = +-1, and
 * exactly c input chunks per compressed chunk in every group) and writes its
 * inverse -- for each compressed chunk, the input chunks the sketch of the
 * SS1 summary page ("Approach") adds into it, with their signs: idx[g][t][0..c-1] are the input chunks of compressed chunk t of
 * group g in ascending order, isign[g][t][r] = sign[g][idx[g][t][r]].
 * Inputs hash[G*J], sign[G*J]; outputs idx[G*Jc*c], isign[G*Jc*c]; all host,
 * caller-owned.  Errors: SS1_ERR_NULL, SS1_ERR_SHAPE, SS1_ERR_PLAN (outputs are
 * then unspecified).
 */
ss1_status ss1_plan_index(const int32_t* hash, const int8_t* sign, int64_t K, int64_t N,
                          int32_t c, int32_t BK, int32_t BN, int32_t* idx, int8_t* isign);

/*
 * ss1_forward -- DEVICE, asynchronous on `stream` (a hipStream_t; NULL means
 * the default stream).  y = SS1(x) for one layer: the input sketch by the
 * plan's signed chunk additions followed by the contraction with W_c (SS1
 * summary page, "Approach").
 *   x   : [M][K]  (rows = M >= 0, cols = K),  dtype F32 or BF16
 *   W_c : [N][K/c], same dtype as x
 *   hash, sign : DEVICE arrays [G][J] as written by ss1_plan (int32 / int8)
 *   y   : [M][N], same dtype as x; written, never read
 * Requirements: K % BK == 0, (K/BK) % c == 0, N % BN == 0, 1 <= c <= SS1_MAX_C,
 * J <= SS1_MAX_CHUNKS; BK % 8 == 0 for BF16 and BK % 4 == 0 for F32; x, W_c and
 * y 16-byte aligned; hash 4-byte aligned.  M == 0 enqueues nothing.
 * The plan must be balanced (as ss1_plan makes it and ss1_plan_index checks);
 * the kernels never read or write outside the buffers whatever the plan
 * holds, but y is unspecified for a plan that is not balanced.
 * Errors: SS1_ERR_NULL, SS1_ERR_SHAPE, SS1_ERR_DTYPE, SS1_ERR_ALIGN (all before
 * any HIP call), SS1_ERR_HIP.
 */
ss1_status ss1_forward(const ss1_tensor* x, const ss1_tensor* W_c,
                       const int32_t* hash, const int8_t* sign,
                       int32_t c, int32_t BK, int32_t BN,
                       ss1_tensor* y, void* stream);

/*
 * ss1_forward_idx -- as ss1_forward, but the plan is given as its inverse
 * index (DEVICE arrays idx [G][Jc][c] int32 and isign [G][Jc][c] int8, as
 * written by ss1_plan_index), which the kernels read directly.  idx must be
 * 4-byte aligned.  Entries outside [0, J) are treated as absent sources.
 */
ss1_status ss1_forward_idx(const ss1_tensor* x, const ss1_tensor* W_c,
                           const int32_t* idx, const int8_t* isign,
                           int32_t c, int32_t BK, int32_t BN,
                           ss1_tensor* y, void* stream);

/*
 * ss1_forward_algo / ss1_forward_idx_algo -- as ss1_forward / ss1_forward_idx
 * with an explicit kernel choice (ss1_algo).  Returns SS1_ERR_ALGO, before any
 * HIP call, when that kernel cannot run the given dtype or shape:
 *   FUSED  : BF16, BK % 32 == 0, BN in {32, 64, 128}
 *   SMALLM : BF16, M <= 16, BK % 32 == 0, BN % 16 == 0
 *   GEMV   : BF16, M <= 4, BN % 16 == 0, 512 <= Kc = K/c <= 65536 (32768
 *            for M = 2, 4096 for M = 3 or 4), and K/BK <= 2 T, where
 *            T = 64 ceil(Kc / (512 Q)) threads take Q = 1 (Kc <= 8192), 2, 4
 *            or 8 slices of 8 compressed columns each.  Each block's weight
 *            loads are all issued before it waits for anything.
 *   DECODE : BF16, M <= 16, K % 512 == 0, BN in {32, 64}, BK % 32 == 0,
 *            K/BK <= 2048, and 16 rows of K bf16 plus the group's plan fit
 *            in one block's LDS (K up to 4096 on gfx950).  One block per
 *            neuron group: the input rows go to LDS once, every weight load
 *            of a wave is issued before it waits, the sketch rounded to bf16
 *            feeds bf16 MFMAs (the same y as SMALLM up to summation order).
 *   GENERIC: any valid call
 *   BAND   : BF16, BK % 32 == 0, BN in {32, 64, 128}, and 32 input rows of K
 *            bf16 (plus the plan) fit in one block's LDS (K up to about 2400)
 *   FOLD   : BF16, BK % 64 == 0, and N a multiple of 128 (or 256) that BN
 *            divides into whole groups; 256*K and 256*Kc under 2^30 elements.
 *            Multiplies x by the expanded weight W_c S_g (built in LDS from
 *            W_c, never stored): the same y as the sketch kernels up to
 *            rounding (no bf16 rounding of a sketch), dense MFMA work.
 *   GROUP  : BF16 weights, c in {2, 4, 8}, BK % 64 == 0, BN in {64, 128}, and
 *            the block's stages fit in LDS (true for every such layer on
 *            gfx950).  One neuron group and 64-256 tokens per block: only the
 *            compressed contraction (2 M N K / c) plus the sketch, which is
 *            formed on the matrix cores (two signed sources per bf16 MFMA) and
 *            rounded to bf16 as in the sketch kernels.  Never picked by
 *            ss1_forward: its per-group gather of x makes it slower than FOLD
 *            on the large-M layers measured.  (SS1 summary page, "Approach":
 *            the sketch cuts the multiplies by c.)
 * ss1_forward picks GEMV for M <= 4 where it applies, else DECODE, else
 * SMALLM for M <= 16, and FOLD for large M where its modelled time is below the sketch
 * kernels' (ss1_select_algo reports the choice).
 * Reproducibility: a row of y depends only on that row of x, but its bits
 * depend on the kernel that runs, and the choice depends on M (and on the
 * device's compute-unit count and LDS size).  Calls with the same M on the
 * same device give identical bits; the same row in calls of different M may
 * differ within the documented rounding (the fold rounds no sketch, the
 * sketch kernels do, and the small-M kernels sum k in another order).
 */
ss1_status ss1_forward_algo(const ss1_tensor* x, const ss1_tensor* W_c,
                            const int32_t* hash, const int8_t* sign,
                            int32_t c, int32_t BK, int32_t BN,
                            ss1_tensor* y, int32_t algo, void* stream);
ss1_status ss1_forward_idx_algo(const ss1_tensor* x, const ss1_tensor* W_c,
                                const int32_t* idx, const int8_t* isign,
                                int32_t c, int32_t BK, int32_t BN,
                                ss1_tensor* y, int32_t algo, void* stream);

/*
 * ss1_select_algo -- HOST.  The kernel (an ss1_algo value, never AUTO) that
 * ss1_forward would run for a layer with these descriptors; only their
 * dtypes and sizes are read (data may be NULL).  With W_c of dtype
 * FP8_E4M3 (and x BF16) it reports the kernel ss1_forward_fp8w would run
 * (GEMV, SMALLM, FOLD or FUSED).  For M == 0 it reports the kernel a non-empty call
 * of the same layer would use.  May query the current HIP device's
 * properties.  Errors: as the shape and dtype checks of ss1_forward (of
 * ss1_forward_fp8w for E4M3 weights).
 */
ss1_status ss1_select_algo(const ss1_tensor* x, const ss1_tensor* W_c, int32_t c, int32_t BK,
                           int32_t BN, int32_t* algo);

/*
 * ss1_forward_ws_query -- HOST.  For a layer with these descriptors (only
 * dtypes and sizes are read; data may be NULL): *algo = the kernel
 * ss1_forward_ws runs and *bytes = the device workspace it needs (0 when it
 * needs none).  SS1_ALGO_SPLIT needs Q * M * N * 4 bytes, Q the number of
 * column slices per neuron group; every other choice is ss1_forward's and
 * needs none.  May query the current HIP device's properties.  Errors: as
 * the shape and dtype checks of ss1_forward, SS1_ERR_NULL.
 *
 * ss1_forward_ws -- DEVICE, asynchronous on `stream`.  ss1_forward with a
 * caller-owned device workspace, which lets decode shapes (5 <= M <= 16,
 * BF16, BN of 32 or 64, BK % 64 == 0) whose input rows are too long for the
 * DECODE kernel (16 rows of K bf16 over one block's LDS) split each neuron
 * group's compressed columns over several blocks (SS1_ALGO_SPLIT): the fewest
 * slices Q (a power of two, K % (512 Q) == 0, Kc % (BK Q) == 0) that give a
 * block per compute unit and fit in LDS.  One block per (group, slice)
 * stages only the input chunks its slice's compressed chunks sum (SS1
 * summary page, "Approach": the sketch is a signed sum of input chunks, so a
 * slice of the sketch needs only those chunks), multiplies the sketch rounded
 * to bf16 by its slice of W_c on the matrix cores, and writes a float32
 * partial tile; a second kernel sums the slices in a fixed order into y.
 * Where the split does not apply the call runs exactly as ss1_forward and
 * the workspace is not touched.
 *   x, W_c, hash, sign, c, BK, BN, y : as ss1_forward
 *   workspace       : DEVICE, at least the bytes ss1_forward_ws_query reports,
 *                     16-byte aligned; its contents on entry are ignored and
 *                     unspecified afterwards (may be NULL when it needs none)
 *   workspace_bytes : its size
 * Calls that share a workspace must be ordered (one stream).  The result
 * equals ss1_forward's up to float32 summation order.  Errors: as
 * ss1_forward; SS1_ERR_NULL (workspace needed and NULL), SS1_ERR_ALIGN,
 * SS1_ERR_SHAPE (workspace_bytes too small) before any HIP call.
 */
ss1_status ss1_forward_ws_query(const ss1_tensor* x, const ss1_tensor* W_c, int32_t c, int32_t BK, int32_t BN,
                                size_t* bytes, int32_t* algo);
ss1_status ss1_forward_ws(const ss1_tensor* x, const ss1_tensor* W_c, const int32_t* hash, const int8_t* sign,
                          int32_t c, int32_t BK, int32_t BN, ss1_tensor* y, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * ss1_sketch -- DEVICE, asynchronous.  The standalone input sketch (the first
 * of the two steps on the SS1 summary page, "Approach") for every group:
 *   z[g][m][k'] for g < G = N/BN, m < M, k' < Kc, written as a [G*M][Kc]
 *   row-major matrix (z->rows = G*M, z->cols = K/c).
 * x is F32 or BF16; z is F32 (the float32 sum itself) or BF16 (that sum
 * rounded to nearest, ties to even).  F32 x requires F32 z.  hash/sign as for
 * ss1_forward; same alignment rules.
 */
ss1_status ss1_sketch(const ss1_tensor* x, const int32_t* hash, const int8_t* sign,
                      int32_t c, int32_t BK, int32_t BN, int64_t N,
                      ss1_tensor* z, void* stream);

/*
 * ss1_project -- DEVICE, asynchronous on `stream`.  Projects a dense weight
 * onto the SS1 sharing pattern, the step that turns a pre-trained layer into
 * an SS1 layer (the SS1 author abstract: pre-trained models can be projected
 * onto SS1; the summary page's "Key results" use projected BERT and
 * Llama-3-8B layers).  The pages give no formula; the projection here is the
 * least-squares one: for row n of group g = n/BN,
 *   W_c[n][t*BK + u] = (1/c) * sum over the c sources j of compressed chunk t
 *                      of sign[g][j] * W[n][j*BK + u],
 * the mean of the signed dense entries that the shared entry stands for.
 *   W   : [N][K] row-major, F32 or BF16 (N = W->rows, K = W->cols); read only
 *   hash, sign : DEVICE arrays [G][J] as written by ss1_plan; the plan must be
 *         balanced (W_c is unspecified otherwise, but nothing outside the
 *         buffers is touched)
 *   W_c : [N][K/c], same dtype as W; written
 * Arithmetic: the c signed sources summed in float32 in ascending chunk order,
 * divided by c (IEEE division, nearest), rounded to W_c's dtype (bf16: nearest,
 * ties to even).  Requirements: as ss1_forward's chunking rules, BK % 8 == 0
 * for BF16 and % 4 for F32, G <= 65535, W and W_c 16-byte aligned, hash
 * 4-byte aligned.  The caller owns every buffer.
 * Errors: SS1_ERR_NULL, SS1_ERR_SHAPE, SS1_ERR_DTYPE, SS1_ERR_ALIGN (before
 * any HIP call), SS1_ERR_HIP.
 */
ss1_status ss1_project(const ss1_tensor* W, const int32_t* hash, const int8_t* sign,
                       int32_t c, int32_t BK, int32_t BN,
                       ss1_tensor* W_c, void* stream);

/*
 * ss1_mlp_forward -- DEVICE, asynchronous on `stream`.  The SS1 MLP pair of a
 * transformer block (the SS1 summary page's GPT-2 results replace its linear
 * layers; "Measured effects": GPT-2 M/L end-to-end latency with SS1 layers):
 *   h = GELU(SS1_up(x)),  y = SS1_down(h),
 * with GELU in its erf form v * Phi(v) = 0.5 * v * (1 + erf(v / sqrt(2))),
 * applied to the float32 accumulator of the up-projection before h is
 * rounded to its dtype (erf by Abramowitz & Stegun 7.1.26, absolute error
 * at most 1.5e-7).  Each projection is computed as by ss1_forward.
 *   x    : [M][K]               F32 or BF16 (all tensors share the dtype)
 *   up   : W_c [N1][K/c1], plan of a K -> N1 layer
 *   down : W_c [N2][N1/c2], plan of an N1 -> N2 layer
 *   h    : [R][N1] workspace, 1 <= R (R = h->rows; any R when M == 0): the
 *          rows of x are processed in chunks of R, each chunk's h written
 *          here and read back by the down-projection.  A chunk of a few
 *          thousand rows keeps h inside the device's last-level cache
 *          instead of a full [M][N1] round trip through HBM; with R >= M, h
 *          holds GELU(SS1_up(x)) for every row when the call completes.
 *   y    : [M][N2], written
 * Requirements: each layer as for ss1_forward (chunking, alignment of x, h, y
 * and both W_c to 16 bytes, hash 4-byte aligned, balanced plans); x, h and y
 * must not overlap.  M == 0 enqueues nothing.
 * Reproducibility: each chunk's projections run the kernels ss1_forward would
 * pick for that chunk's row count, so y is bit-reproducible for a fixed M and
 * R; another R can change the kernels (ss1_forward's note).
 * Errors: SS1_ERR_NULL, SS1_ERR_SHAPE, SS1_ERR_DTYPE, SS1_ERR_ALIGN (every
 * check runs for both layers before any HIP call), SS1_ERR_HIP.
 */
ss1_status ss1_mlp_forward(const ss1_tensor* x, const ss1_layer* up, const ss1_layer* down,
                           ss1_tensor* h, ss1_tensor* y, void* stream);

/* Bytes of the library's static device workspace used by
   ss1_mlp_forward_static (one array per GPU, held until the process ends). */
#define SS1_STATIC_SCRATCH_BYTES (32u << 20)

/*
 * ss1_mlp_forward_static -- DEVICE, asynchronous on `stream`.  ss1_mlp_forward
 * with no workspace argument and no allocation of any kind, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  h lives in a static device array of
 * SS1_STATIC_SCRATCH_BYTES that the library holds on every GPU it runs on;
 * its device address is looked up once per device (hipGetSymbolAddress) on
 * the first call made there.  The rows are processed in chunks of
 *   R = floor(SS1_STATIC_SCRATCH_BYTES / (N1 * e))   (e = 2 for BF16, 4 for F32),
 * rounded down to a multiple of 256 when R >= 256 -- the same result as
 * ss1_mlp_forward with an h of R rows.  h is written by each chunk's
 * up-projection before its down-projection reads it, so nothing needs
 * clearing; its contents after a call are unspecified.
 *   x, up, down, y : as ss1_mlp_forward
 * Calls that overlap on one GPU (on different streams, or from several host
 * threads) race on the shared array; serialise them.
 * Errors: as ss1_mlp_forward, plus SS1_ERR_SHAPE when one row of h (N1 * e
 * bytes) exceeds SS1_STATIC_SCRATCH_BYTES (checked before any HIP call), and
 * SS1_ERR_HIP when the device or the array's address cannot be obtained.
 * M == 0 checks the descriptors and makes no HIP call.
 */
ss1_status ss1_mlp_forward_static(const ss1_tensor* x, const ss1_layer* up, const ss1_layer* down, ss1_tensor* y,
                                  void* stream);

/*
 * ss1_quantize_fp8 -- DEVICE, asynchronous on `stream`.  Per-row fp8
 * quantization of a compressed weight, for ss1_forward_fp8w.  The SS1
 * summary page ("Measured effects") quantizes SS1 models after training and
 * finds quality unchanged; its "Limitations" say quantized SS1 kernels were
 * not implemented.  This library's scheme (a reading; the pages fix none):
 *   scale[n] = max_k |W_c[n][k]| / 448   (float32 IEEE division; 1 when the
 *                                         row is all zero)
 *   Q[n][k]  = the OCP E4M3 code nearest to W_c[n][k] / scale[n]
 *              (float32 division, ties to even; 448 is E4M3's largest value)
 * so that W_c[n][k] ~= e4m3(Q[n][k]) * scale[n].
 *   W_c   : [N][Kc] BF16 or F32, read
 *   Q     : [N][Kc] SS1_FP8_E4M3, written
 *   scale : DEVICE float[N], written
 * Requirements: Kc even, W_c and Q 16-byte aligned, scale 4-byte aligned;
 * finite inputs.  N == 0 enqueues nothing.
 * Errors: SS1_ERR_NULL, SS1_ERR_SHAPE, SS1_ERR_DTYPE, SS1_ERR_ALIGN (before
 * any HIP call), SS1_ERR_HIP.
 */
ss1_status ss1_quantize_fp8(const ss1_tensor* W_c, ss1_tensor* Q, float* scale, void* stream);

/*
 * ss1_forward_fp8w -- DEVICE, asynchronous on `stream`.  ss1_forward with the
 * compressed weight in fp8 (ss1_quantize_fp8's Q and scale): the layer
 * computed is SS1 with W_c[n][k'] = e4m3(Q[n][k']) * scale[n].  The sketch is
 * formed as in ss1_forward (float32 sum rounded to bf16); each E4M3 weight is
 * converted to bf16 exactly, the products are accumulated in float32 by the
 * bf16 MFMA, and the row's scale multiplies the float32 sum before the bf16
 * rounding of y.  Halves the weight bytes each call reads, which is what
 * bounds small-M (decode) calls.  Kernels: matrix-vector and small-M for
 * decode shapes; the fold, the band kernel (layers whose input rows fit in
 * LDS; c in {1, 2, 4, 8}) or the fused kernel otherwise, chosen as for
 * ss1_forward.
 *   x : [M][K] BF16;  Q : [N][K/c] SS1_FP8_E4M3;  scale : DEVICE float[N];
 *   hash, sign : as ss1_forward;  y : [M][N] BF16, written
 * Requirements: as ss1_forward, plus BK % 32 == 0 and either M <= 16 with
 * BN % 16 == 0, or BN in {32, 64, 128}; scale 4-byte aligned.
 * Errors: as ss1_forward (SS1_ERR_SHAPE for a shape no fp8 kernel takes).
 */
ss1_status ss1_forward_fp8w(const ss1_tensor* x, const ss1_tensor* Q, const float* scale,
                            const int32_t* hash, const int8_t* sign,
                            int32_t c, int32_t BK, int32_t BN,
                            ss1_tensor* y, void* stream);

/*
 * ss1_forward_fp8 -- DEVICE, asynchronous on `stream`.  The SS1 layer with
 * both operands quantized to fp8 and contracted on the fp8 matrix cores (the
 * SS1 summary page, "Limitations": quantized SS1 kernels were not built;
 * "Measured effects": SS1 models quantized after training keep their
 * quality; the SS1 author abstract: SS1 combines with quantization).  The
 * layer computed (a reading; the pages fix no scheme):
 *   y[m][n] = xscale[m] * wscale[n] * sum_k e4m3(xq[m][k]) * sign_g(j) *
 *             e4m3(Wq[n][h_g(j)*BK + u])      (k = j*BK + u, g = n / BN)
 * i.e. SS1 of the dequantized input and weight.  Each product of two E4M3
 * values is exact in float32, the sums accumulate in float32 on the MFMA
 * (v_mfma_scale_f32_16x16x128_f8f6f4, unit block scales), the two row
 * scales multiply the sum, and y is rounded to bf16 (nearest, ties to even).
 * Quantize x per row with ss1_quantize_fp8 (one scale per token row) and W_c
 * per row likewise.  The kernel multiplies x by the expanded weight (no
 * sketch is formed), dense MFMA work at twice the bf16 rate.
 *   xq : [M][K] SS1_FP8_E4M3;  xscale : DEVICE float[M]
 *   Wq : [N][K/c] SS1_FP8_E4M3;  wscale : DEVICE float[N]
 *   hash, sign : as ss1_forward;  y : [M][N] BF16, written
 * Requirements: ss1_forward's chunking, plus N % 256 == 0, 256 % BN == 0,
 * BK % 64 == 0, K % 128 == 0, 256*K and N*K/c under 2^31; xq, Wq and y
 * 16-byte aligned, scales 4-byte aligned.  M == 0 enqueues nothing.
 * Errors: SS1_ERR_NULL, SS1_ERR_DTYPE, SS1_ERR_SHAPE, SS1_ERR_ALIGN (before
 * any HIP call), SS1_ERR_HIP.
 */
ss1_status ss1_forward_fp8(const ss1_tensor* xq, const float* xscale, const ss1_tensor* Wq, const float* wscale,
                           const int32_t* hash, const int8_t* sign, int32_t c, int32_t BK, int32_t BN,
                           ss1_tensor* y, void* stream);

/*
 * ss1_backward -- DEVICE, asynchronous on `stream`.  Gradients of
 * y = ss1_forward(x, W_c) for an upstream gradient dy (the SS1 summary page,
 * "Limitations": the backward pass is not reduced, it costs what a dense
 * layer's does):
 *   dW_c[g-block] = dy[:, g-block]^T z_g        (z_g: group g's sketch of x)
 *   dx[:, j-chunk] = sum over groups g of sign[g][j] *
 *                    (dy[:, g-block] W_c[g-block])[:, hash[g][j]-chunk]
 * (dx = dy times the dense weight SS1 stands for).  z_g is formed as in
 * ss1_forward (float32 sum of the signed sources, rounded to bf16); products
 * accumulate in float32 on the bf16 MFMA; outputs are rounded to bf16.
 *   x  : [M][K] BF16;  W_c : [N][K/c] BF16;  hash, sign : as ss1_forward
 *   dy : [M][N] BF16, read
 *   dx : [M][K] BF16, written (NULL: not computed)
 *   dW_c : [N][K/c] BF16, written (NULL: not computed; all zero when M == 0)
 * Requirements: ss1_forward's, plus BF16 only, BK % 32 == 0, BN % 32 == 0,
 * G <= 8192.  All buffers 16-byte aligned.  The caller owns every buffer.
 * Errors: SS1_ERR_NULL, SS1_ERR_SHAPE, SS1_ERR_DTYPE, SS1_ERR_ALIGN (before
 * any HIP call), SS1_ERR_HIP.
 */
ss1_status ss1_backward(const ss1_tensor* x, const ss1_tensor* W_c,
                        const int32_t* hash, const int8_t* sign,
                        int32_t c, int32_t BK, int32_t BN,
                        const ss1_tensor* dy, ss1_tensor* dx, ss1_tensor* dW_c,
                        void* stream);

/*
 * ss1_backward_select_algo -- HOST.  The kernels ss1_backward runs for these
 * descriptors (only dtypes and sizes are read; data may be NULL):
 *   *dw_algo = SS1_ALGO_FOLD  : dW_c contracted over (token, source) with no
 *                               sketch formed -- the exact sum, rounded once
 *              SS1_ALGO_FUSED : dW_c from the group's sketch rounded to bf16
 *                               (as the forward's sketch kernels form it)
 *   *dx_algo = SS1_ALGO_FOLD or SS1_ALGO_GENERIC (tiled dx kernels); neither
 *              forms a sketch, both round only dx itself.
 * For M == 0 it reports what a non-empty call of the same layer would use.
 * May query the current HIP device's properties (LDS size).
 * Errors: as the shape and dtype checks of ss1_backward.
 */
ss1_status ss1_backward_select_algo(const ss1_tensor* x, const ss1_tensor* W_c, int32_t c, int32_t BK,
                                    int32_t BN, int32_t* dx_algo, int32_t* dw_algo);

#ifdef __cplusplus
}
#endif

#endif /* SS1_H */
