"""Plain CPU oracle for the Sketch Structured Transform (SS1) linear-layer forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its Python binding) never touches it, and it
shares no code with that path: not the plan generator, not the bf16 decoding,
not the index construction.  Random numbers the method draws (the hash and the
signs) come from SplitMix64, a published counter-based generator that this
module implements on its own from its definition.

What it computes, and where that is stated
------------------------------------------
Sources (page titles; no code exists on any of them):

* "SS1: Accelerating Inference with Fast and Expressive Sketch Structured
  Transform" (atlas.scime.ai summary page), section *Approach*: parameter
  sharing is confined to each neuron's own weight vector; hash functions that
  are coalesced along K and along N make the layer first sketch its input down
  by the compression factor with additions and subtractions only, and then
  multiply that sketch by the compressed weight, so FLOPs drop by the factor.
* The SS1 author abstract (taxoreview abstract list for that author group):
  the operator shares parameters randomly but in a structured way to cut
  computation; dense pre-trained layers can be projected onto it.
* CountSketch (Charikar, Chen and Farach-Colton 2002, entry 29 of the reference
  list on the "Deja Vu: Contextual Sparsity" page): a sketch that adds each
  coordinate, with a random sign, into one random bucket.

Readings where the pages are silent (each is listed in the design doc):

* K-coalescing: inputs are cut into J = K/BK chunks of BK consecutive
  coordinates; input chunk j of neuron group g lands in compressed chunk
  hash[g][j], keeping its offset u inside the chunk.
* N-coalescing: BN consecutive neurons (group g = n // BN) share one hash and
  one sign vector; groups are independent.
* Signs: one +-1 per (group, input chunk); no scaling by 1/sqrt(c); no bias.
* Balanced hash: every compressed chunk receives exactly c input chunks.  The
  oracle's forward accepts any hash in range (balanced or not); only the plan
  generator promises balance.
* Plan generator: SplitMix64, Fisher-Yates with plain modulo, then one sign bit
  per chunk (top bit of a draw), all per group in group order.
* Precision: everything in float64; bf16 inputs are widened exactly.
* Projection of a dense weight onto SS1 (the pages only say that pre-trained
  layers can be projected): least squares onto the sharing pattern, i.e. each
  compressed entry is the mean of its signed sources.

Nothing here is blocked, fused or reordered beyond the definition.
"""
from __future__ import annotations

import math

import numpy as np

_MASK64 = (1 << 64) - 1
_GOLDEN_GAMMA = 0x9E3779B97F4A7C15


class SplitMix64:
    """SplitMix64 (Steele, Lea and Flood, OOPSLA 2014, "Fast splittable
    pseudorandom number generators"), as published by its authors: the state
    advances by the golden-ratio gamma and each output is the state passed
    through a 64-bit xor-shift-multiply finaliser.  Python integers, masked to
    64 bits, so every step is exact."""

    def __init__(self, seed: int):
        self.state = int(seed) & _MASK64

    def next(self) -> int:
        self.state = (self.state + _GOLDEN_GAMMA) & _MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        return z ^ (z >> 31)


def dims(K: int, N: int, c: int, BK: int, BN: int) -> dict:
    """Derived sizes: J input chunks, Jc compressed chunks, Kc compressed width,
    G neuron groups.  Raises ValueError when the chunking does not divide."""
    if min(K, N, c, BK, BN) <= 0:
        raise ValueError("K, N, c, BK, BN must be positive")
    if K % BK:
        raise ValueError("K must be a multiple of BK")
    J = K // BK
    if J % c:
        raise ValueError("the number of input chunks K/BK must be a multiple of c")
    if N % BN:
        raise ValueError("N must be a multiple of BN")
    Jc = J // c
    return {"J": J, "Jc": Jc, "Kc": Jc * BK, "G": N // BN}


def plan(seed: int, K: int, N: int, c: int, BK: int, BN: int):
    """Seeded balanced chunk hash and +-1 signs, one pair of vectors per group.

    Group by group, in order: shuffle the J chunk ids with Fisher-Yates (for
    i = J-1 down to 1, swap position i with position ``draw % (i+1)``); the
    shuffled list is cut into Jc consecutive runs of c and run t becomes the
    source set of compressed chunk t.  Then draw one value per input chunk,
    in chunk order, and use its top bit as the sign (1 -> -1).

    Returns ``hash`` int32 [G][J] with values in [0, Jc) and ``sign`` int8
    [G][J] with values +-1."""
    d = dims(K, N, c, BK, BN)
    J, G = d["J"], d["G"]
    rng = SplitMix64(seed)
    hash_ = np.empty((G, J), dtype=np.int32)
    sign = np.empty((G, J), dtype=np.int8)
    for g in range(G):
        order = list(range(J))
        for i in range(J - 1, 0, -1):
            k = rng.next() % (i + 1)
            order[i], order[k] = order[k], order[i]
        for p in range(J):
            hash_[g, order[p]] = p // c
        for j in range(J):
            sign[g, j] = -1 if (rng.next() >> 63) else 1
    return hash_, sign


def identity_plan(K: int, N: int, BK: int, BN: int):
    """The c = 1 plan that maps every chunk to itself with sign +1, under which
    SS1 must reduce to a dense linear layer (the zero-compression end of the
    parameter-sharing family)."""
    d = dims(K, N, 1, BK, BN)
    J, G = d["J"], d["G"]
    hash_ = np.tile(np.arange(J, dtype=np.int32), (G, 1))
    sign = np.ones((G, J), dtype=np.int8)
    return hash_, sign


def check_plan(hash_, sign, K: int, N: int, c: int, BK: int, BN: int, balanced: bool = True):
    """Validate a plan: shapes, 0 <= hash < Jc, sign in {-1, +1}, and (when
    ``balanced``) exactly c input chunks per compressed chunk in every group.
    Raises ValueError naming the first violation."""
    d = dims(K, N, c, BK, BN)
    J, Jc, G = d["J"], d["Jc"], d["G"]
    hash_ = np.asarray(hash_)
    sign = np.asarray(sign)
    if hash_.shape != (G, J) or sign.shape != (G, J):
        raise ValueError(f"plan arrays must have shape {(G, J)}")
    for g in range(G):
        counts = [0] * Jc
        for j in range(J):
            t = int(hash_[g, j])
            if not 0 <= t < Jc:
                raise ValueError(f"hash[{g}][{j}] = {t} outside [0, {Jc})")
            if int(sign[g, j]) not in (-1, 1):
                raise ValueError(f"sign[{g}][{j}] = {int(sign[g, j])} is not +-1")
            counts[t] += 1
        if balanced:
            for t in range(Jc):
                if counts[t] != c:
                    raise ValueError(f"group {g}: compressed chunk {t} receives {counts[t]} chunks, not {c}")


def plan_index(hash_, sign, K: int, N: int, c: int, BK: int, BN: int):
    """Inverse of a balanced plan: ``idx[g][t]`` lists the c input chunks that
    land in compressed chunk t of group g, in ascending order, and
    ``isign[g][t][r]`` is the sign of ``idx[g][t][r]``.  int32 and int8 arrays
    of shape [G][Jc][c]."""
    check_plan(hash_, sign, K, N, c, BK, BN, balanced=True)
    d = dims(K, N, c, BK, BN)
    J, Jc, G = d["J"], d["Jc"], d["G"]
    idx = np.empty((G, Jc, c), dtype=np.int32)
    isign = np.empty((G, Jc, c), dtype=np.int8)
    for g in range(G):
        fill = [0] * Jc
        for j in range(J):  # ascending j gives ascending sources per slot
            t = int(hash_[g, j])
            idx[g, t, fill[t]] = j
            isign[g, t, fill[t]] = sign[g, j]
            fill[t] += 1
    return idx, isign


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly: a bf16 value is the float32
    whose top 16 bits are the pattern and whose low 16 bits are zero."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def sketch(x, hash_, sign, K: int, N: int, c: int, BK: int, BN: int, dtype=np.float64) -> np.ndarray:
    """Per-group chunk sketch of the input rows, in float64.

    For every group g a fresh [M][Kc] accumulator starts at zero; walking the
    input chunks j in ascending order, chunk j of every row, times sign[g][j],
    is added into compressed chunk hash[g][j] at the same offsets.  Returns
    z with shape [G][M][Kc].  Accepts any in-range hash (balance not needed).
    ``dtype`` float32 runs the same steps in float32 (only the CPU-speed
    baseline of the benchmark uses it; the definition is float64)."""
    d = dims(K, N, c, BK, BN)
    J, Kc, G = d["J"], d["Kc"], d["G"]
    x = np.asarray(x, dtype=dtype)
    if x.ndim != 2 or x.shape[1] != K:
        raise ValueError(f"x must have shape [M][{K}]")
    check_plan(hash_, sign, K, N, c, BK, BN, balanced=False)
    M = x.shape[0]
    z = np.zeros((G, M, Kc), dtype=dtype)
    for g in range(G):
        for j in range(J):
            t = int(hash_[g, j])
            s = dtype(sign[g, j])
            z[g, :, t * BK:(t + 1) * BK] += s * x[:, j * BK:(j + 1) * BK]
    return z


def forward(x, Wc, hash_, sign, K: int, N: int, c: int, BK: int, BN: int, dtype=np.float64) -> np.ndarray:
    """SS1 forward in float64: sketch the input (as in :func:`sketch`), then
    multiply group g's sketch by its BN rows of the compressed weight,
    ``y[:, g*BN:(g+1)*BN] = z_g @ Wc[g*BN:(g+1)*BN, :].T``.

    ``x`` is [M][K], ``Wc`` is [N][Kc] (row-major, one row per neuron, like a
    dense linear layer's [out][in] weight).  Returns y, [M][N] float64
    (``dtype`` float32: the same steps in float32, for the benchmark's
    CPU-speed baseline only)."""
    d = dims(K, N, c, BK, BN)
    Kc, G = d["Kc"], d["G"]
    Wc = np.asarray(Wc, dtype=dtype)
    if Wc.shape != (N, Kc):
        raise ValueError(f"Wc must have shape {(N, Kc)}")
    z = sketch(x, hash_, sign, K, N, c, BK, BN, dtype=dtype)
    M = z.shape[1]
    y = np.empty((M, N), dtype=dtype)
    for g in range(G):
        y[:, g * BN:(g + 1) * BN] = z[g] @ Wc[g * BN:(g + 1) * BN, :].T
    return y


def dense_expand(Wc, hash_, sign, K: int, N: int, c: int, BK: int, BN: int) -> np.ndarray:
    """The dense [N][K] weight that SS1's parameter sharing stands for: entry
    (n, j*BK + u) is sign[g][j] * Wc[n, hash[g][j]*BK + u] with g = n // BN.
    By linearity ``x @ dense_expand(...).T`` equals :func:`forward`."""
    d = dims(K, N, c, BK, BN)
    J, Kc, G = d["J"], d["Kc"], d["G"]
    Wc = np.asarray(Wc, dtype=np.float64)
    if Wc.shape != (N, Kc):
        raise ValueError(f"Wc must have shape {(N, Kc)}")
    check_plan(hash_, sign, K, N, c, BK, BN, balanced=False)
    W = np.empty((N, K), dtype=np.float64)
    for g in range(G):
        rows = slice(g * BN, (g + 1) * BN)
        for j in range(J):
            t = int(hash_[g, j])
            W[rows, j * BK:(j + 1) * BK] = float(sign[g, j]) * Wc[rows, t * BK:(t + 1) * BK]
    return W


def sketch_rounded(x, hash_, sign, K: int, N: int, c: int, BK: int, BN: int,
                   to_bf16: bool) -> np.ndarray:
    """Diagnostic "mirror" sketch: the same sum as :func:`sketch`, but taken in
    float32 over the sources of each compressed chunk in ascending chunk order
    (starting from the first signed source), then, when ``to_bf16``, rounded
    to the nearest bf16 value with ties to even.  A GPU path that keeps its
    sketch in float32 and rounds it to bf16 once should reproduce this bit for
    bit for c <= 2 and closely otherwise.  Returns float64 values of the
    rounded sketch, [G][M][Kc]."""
    d = dims(K, N, c, BK, BN)
    J, Jc, Kc, G = d["J"], d["Jc"], d["Kc"], d["G"]
    x32 = np.asarray(x, dtype=np.float32)
    M = x32.shape[0]
    check_plan(hash_, sign, K, N, c, BK, BN, balanced=False)
    z = np.zeros((G, M, Kc), dtype=np.float64)
    for g in range(G):
        acc = [None] * Jc
        for j in range(J):
            t = int(hash_[g, j])
            term = np.float32(sign[g, j]) * x32[:, j * BK:(j + 1) * BK]
            acc[t] = term if acc[t] is None else (acc[t] + term).astype(np.float32)
        for t in range(Jc):
            if acc[t] is None:
                continue
            v = acc[t]
            if to_bf16:
                v = _round_f32_to_bf16(v)
            z[g, :, t * BK:(t + 1) * BK] = v.astype(np.float64)
    return z


def _round_f32_to_bf16(v) -> np.ndarray:
    """Round float32 values to bf16 precision (8 significant bits), nearest,
    ties to even, computed on the float64 value with frexp/ldexp so that no
    bit trick is shared with any other code.  Finite inputs only."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)              # v = m * 2**e, 0.5 <= |m| < 1
    scaled = np.ldexp(m, 8)         # 8 significant bits left of the point
    r = np.round(scaled)            # numpy rounds half to even
    return np.ldexp(r, e - 8).astype(np.float32)


def forward_mirror(x, Wc, hash_, sign, K: int, N: int, c: int, BK: int, BN: int,
                   sketch_bf16: bool) -> np.ndarray:
    """Diagnostic forward using :func:`sketch_rounded` (float32 sketch, then
    optionally bf16) followed by the same float64 contraction as
    :func:`forward`.  Used for a tighter check than the plain tolerance."""
    d = dims(K, N, c, BK, BN)
    Kc, G = d["Kc"], d["G"]
    Wc = np.asarray(Wc, dtype=np.float64)
    if Wc.shape != (N, Kc):
        raise ValueError(f"Wc must have shape {(N, Kc)}")
    z = sketch_rounded(x, hash_, sign, K, N, c, BK, BN, sketch_bf16)
    M = z.shape[1]
    y = np.empty((M, N), dtype=np.float64)
    for g in range(G):
        y[:, g * BN:(g + 1) * BN] = z[g] @ Wc[g * BN:(g + 1) * BN, :].T
    return y


def project(W, hash_, sign, K: int, N: int, c: int, BK: int, BN: int) -> np.ndarray:
    """Projection of a dense [N][K] weight onto SS1's sharing pattern, float64.

    The SS1 author abstract states that pre-trained dense layers can be
    projected onto the operator (and the summary page's *Key results* use such
    projected BERT and Llama-3-8B layers); the pages give no formula.  The
    plain reading taken here is the least-squares projection: for row n of
    group g = n // BN, compressed entry (n, t*BK + u) minimises
    sum over sources j of t of (W[n, j*BK + u] - sign[g][j] * Wc[n, t*BK + u])^2,
    whose minimiser is the mean of sign[g][j] * W[n, j*BK + u] over those
    sources (c of them in a balanced plan).  A compressed chunk with no source
    gets 0 (the minimum-norm solution).  Sources are walked in ascending j.
    Returns Wc, [N][Kc] float64."""
    d = dims(K, N, c, BK, BN)
    J, Jc, Kc, G = d["J"], d["Jc"], d["Kc"], d["G"]
    W = np.asarray(W, dtype=np.float64)
    if W.shape != (N, K):
        raise ValueError(f"W must have shape {(N, K)}")
    check_plan(hash_, sign, K, N, c, BK, BN, balanced=False)
    Wc = np.zeros((N, Kc), dtype=np.float64)
    for g in range(G):
        rows = slice(g * BN, (g + 1) * BN)
        count = np.zeros(Jc, dtype=np.int64)
        for j in range(J):
            t = int(hash_[g, j])
            Wc[rows, t * BK:(t + 1) * BK] += float(sign[g, j]) * W[rows, j * BK:(j + 1) * BK]
            count[t] += 1
        for t in range(Jc):
            if count[t] > 0:
                Wc[rows, t * BK:(t + 1) * BK] /= float(count[t])
    return Wc


def project_rounded(W, hash_, sign, K: int, N: int, c: int, BK: int, BN: int,
                    to_bf16: bool) -> np.ndarray:
    """Diagnostic "mirror" of :func:`project` for a float32 device path: the
    signed sources of each compressed chunk summed in float32 in ascending
    chunk order (from the first signed source), divided by the source count
    in float32 (IEEE division, nearest), then, when ``to_bf16``, rounded to
    the nearest bf16 value with ties to even.  Returns float64 values."""
    d = dims(K, N, c, BK, BN)
    J, Jc, Kc, G = d["J"], d["Jc"], d["Kc"], d["G"]
    W32 = np.asarray(W, dtype=np.float32)
    if W32.shape != (N, K):
        raise ValueError(f"W must have shape {(N, K)}")
    check_plan(hash_, sign, K, N, c, BK, BN, balanced=False)
    Wc = np.zeros((N, Kc), dtype=np.float64)
    for g in range(G):
        rows = slice(g * BN, (g + 1) * BN)
        acc = [None] * Jc
        count = [0] * Jc
        for j in range(J):
            t = int(hash_[g, j])
            term = np.float32(sign[g, j]) * W32[rows, j * BK:(j + 1) * BK]
            acc[t] = term if acc[t] is None else (acc[t] + term).astype(np.float32)
            count[t] += 1
        for t in range(Jc):
            if acc[t] is None:
                continue
            v = (acc[t] / np.float32(count[t])).astype(np.float32)
            if to_bf16:
                v = _round_f32_to_bf16(v)
            Wc[rows, t * BK:(t + 1) * BK] = v.astype(np.float64)
    return Wc


def gelu(v) -> np.ndarray:
    """GELU in its defining form, v * Phi(v) with Phi the standard normal
    distribution function, float64.  Phi is taken as 0.5 * erfc(-v / sqrt(2))
    (the same function as 0.5 * (1 + erf(v / sqrt(2))) without its
    cancellation for large negative v).  The pages name the GPT-2 MLP
    (up-projection, activation, down-projection) without fixing the GELU
    variant; the defining form is the plain reading."""
    v = np.asarray(v, dtype=np.float64)
    erfc = np.vectorize(math.erfc, otypes=[np.float64])
    return v * 0.5 * erfc(-v / math.sqrt(2.0))


def mlp_forward(x, up: dict, down: dict, round_h_to_bf16: bool = False):
    """The SS1 MLP pair: h = GELU(SS1_up(x)), y = SS1_down(h), float64.

    ``up`` and ``down`` hold Wc, hash, sign, K, N, c, BK, BN of each layer
    (down.K == up.N).  With ``round_h_to_bf16`` the intermediate h is rounded
    to bf16 (nearest, ties to even) before the down-projection, as a device
    path that keeps h in bf16 does.  Returns (h, y)."""
    if down["K"] != up["N"]:
        raise ValueError("down.K must equal up.N")
    h = gelu(forward(x, up["Wc"], up["hash"], up["sign"], up["K"], up["N"], up["c"], up["BK"], up["BN"]))
    if round_h_to_bf16:
        h = _round_f32_to_bf16(h.astype(np.float32)).astype(np.float64)
    y = forward(h, down["Wc"], down["hash"], down["sign"], down["K"], down["N"], down["c"], down["BK"],
                down["BN"])
    return h, y


def backward(x, Wc, dy, hash_, sign, K: int, N: int, c: int, BK: int, BN: int):
    """Gradients of the SS1 forward, float64, for y = forward(x, Wc) and an
    upstream gradient dy [M][N].  The summary page's *Limitations* note that
    the backward pass is not reduced; written out from the forward's two
    steps:

    * dWc: y[:, g-block] = z_g @ Wc[g-block].T, so
      dWc[g-block] = dy[:, g-block].T @ z_g (z_g the group's sketch);
    * dx: dz_g = dy[:, g-block] @ Wc[g-block] is the gradient of the sketch,
      and the sketch added sign[g][j] * x-chunk j into chunk hash[g][j], so
      dx-chunk j receives sign[g][j] * dz_g-chunk hash[g][j], summed over
      the groups.

    Returns (dx [M][K], dWc [N][Kc])."""
    d = dims(K, N, c, BK, BN)
    J, Kc, G = d["J"], d["Kc"], d["G"]
    x = np.asarray(x, dtype=np.float64)
    Wc = np.asarray(Wc, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    M = x.shape[0]
    if Wc.shape != (N, Kc) or dy.shape != (M, N):
        raise ValueError("shape mismatch")
    z = sketch(x, hash_, sign, K, N, c, BK, BN)
    dWc = np.empty((N, Kc), dtype=np.float64)
    dx = np.zeros((M, K), dtype=np.float64)
    for g in range(G):
        rows = slice(g * BN, (g + 1) * BN)
        dWc[rows] = dy[:, rows].T @ z[g]
        dz = dy[:, rows] @ Wc[rows]
        for j in range(J):
            t = int(hash_[g, j])
            dx[:, j * BK:(j + 1) * BK] += float(sign[g, j]) * dz[:, t * BK:(t + 1) * BK]
    return dx, dWc


def backward_dw_mirror(x, dy, hash_, sign, K: int, N: int, c: int, BK: int, BN: int) -> np.ndarray:
    """Diagnostic dWc for a device path that rounds the sketch to bf16 (as the
    forward does) before the float32-accumulated product: dy_g.T @ z_g with z
    from :func:`sketch_rounded`, in float64."""
    d = dims(K, N, c, BK, BN)
    G = d["G"]
    z = sketch_rounded(x, hash_, sign, K, N, c, BK, BN, True)
    dy = np.asarray(dy, dtype=np.float64)
    out = np.empty((N, d["Kc"]), dtype=np.float64)
    for g in range(G):
        rows = slice(g * BN, (g + 1) * BN)
        out[rows] = dy[:, rows].T @ z[g]
    return out


# ------------------------------------------------------------- fp8 weights
# OCP 8-bit floating point, E4M3 ("FN": no infinities): 1 sign bit, 4
# exponent bits (bias 7), 3 mantissa bits; exponent field 0 holds subnormals
# m * 2^-9; S.1111.111 is NaN, so the largest finite magnitude is
# 1.75 * 2^8 = 448.  (OCP "OFP8 Formats for Deep Learning", v1.0.)
E4M3_MAX = 448.0


def e4m3_decode(code) -> np.ndarray:
    """Value of each E4M3 code (uint8), float64; NaN for the two NaN codes."""
    code = np.asarray(code, dtype=np.int64)
    sgn = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 0xF
    m = code & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sgn * mag


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 code of each finite value, ties to the even mantissa,
    magnitudes beyond 448 saturated to 448 (uint8).  Walks the value's
    binade: the quantum is 2^(e-3) for |v| in [2^e, 2^(e+1)), e >= -6, and
    2^-9 below 2^-6 (subnormals)."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.uint8)
    for idx, x in np.ndenumerate(v):
        neg = x < 0 or (x == 0 and math.copysign(1.0, x) < 0)
        a = abs(float(x))
        if a == 0.0:
            out[idx] = 0x80 if neg else 0
            continue
        e = max(math.floor(math.log2(a)), -6)
        if 2.0 ** e > a:               # log2 rounding at binade edges
            e -= 1
        elif 2.0 ** (e + 1) <= a:
            e += 1
        e = max(e, -6)
        q = 2.0 ** (e - 3)
        n = a / q                      # exact: a power-of-two scaling
        r = math.floor(n)
        frac = n - r
        if frac > 0.5 or (frac == 0.5 and r % 2 == 1):
            r += 1
        mag = r * q
        if mag > E4M3_MAX:
            mag = E4M3_MAX
        if mag < 2.0 ** -6:            # subnormal (or rounded up to 2^-6)
            code = int(round(mag / 2.0 ** -9))
            code = 0x08 if code == 8 else code
        else:
            ee = math.floor(math.log2(mag))
            mm = int(round((mag / 2.0 ** ee - 1.0) * 8))
            code = ((ee + 7) << 3) | mm
        out[idx] = code | (0x80 if neg else 0)
    return out


def quantize_fp8_rows(Wc):
    """Per-row E4M3 quantization of a compressed weight, as float32 device
    arithmetic does it: scale[n] = max_k |Wc[n, k]| / 448 (float32 division,
    nearest; 1.0 for an all-zero row), q = Wc / scale (float32 division), then
    the nearest E4M3 code.  Returns (codes uint8 [N][Kc], scale float32 [N])."""
    W32 = np.asarray(Wc, dtype=np.float32)
    amax = np.max(np.abs(W32), axis=1).astype(np.float32)
    scale = np.where(amax > 0, (amax / np.float32(E4M3_MAX)).astype(np.float32), np.float32(1.0))
    scale = scale.astype(np.float32)
    q = (W32 / scale[:, None]).astype(np.float32)
    return e4m3_encode(q.astype(np.float64)), scale


def dequantize_fp8_rows(codes, scale) -> np.ndarray:
    """Float64 weight that a quantized layer stands for: code value * scale."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[:, None]


def flops(M: int, K: int, N: int, c: int) -> dict:
    """Work of one forward: the compressed contraction does 2*M*N*K/c FLOPs
    (the reduction by c the method claims); the dense layer it replaces does
    2*M*N*K.  Sketch additions are counted apart: each of the G groups adds
    M*K/c*(c-1) values."""
    return {"compressed": 2 * M * N * K // c, "dense_equiv": 2 * M * N * K}
