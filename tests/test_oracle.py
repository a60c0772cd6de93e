"""Pins for the CPU oracle, each against something other than the oracle itself:
published generator values, brute-force expansion into the equivalent dense
weight, the c = 1 identity case against a library matmul, the Kronecker
(CountSketch-matrix) form, the textbook CountSketch scatter, and invariants of
the plan.  CPU only."""
import itertools
import os

import numpy as np
import pytest

import oracle
from ss1_inputs import bf16_bits_to_f32, draw, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kat():
    out, seed = {}, None
    with open(os.path.join(GOLDEN, "splitmix64_kat.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("seed"):
                seed = int(line.split()[1])
                out[seed] = []
            else:
                out[seed].append(int(line))
    return out


def test_splitmix64_known_answers():
    for seed, vals in _kat().items():
        r = oracle.SplitMix64(seed)
        assert [r.next() for _ in vals] == vals


# ----------------------------------------------------------------- plan pins
SHAPES = [  # K, N, c, BK, BN
    (256, 256, 2, 32, 32),
    (48, 12, 3, 4, 3),
    (48, 8, 4, 2, 2),
    (16, 4, 1, 2, 1),
    (96, 6, 8, 1, 6),
]


@pytest.mark.parametrize("K,N,c,BK,BN", SHAPES)
def test_plan_balanced_and_signed(K, N, c, BK, BN):
    h, s = oracle.plan(7, K, N, c, BK, BN)
    d = oracle.dims(K, N, c, BK, BN)
    assert h.shape == (d["G"], d["J"]) and s.shape == (d["G"], d["J"])
    assert h.dtype == np.int32 and s.dtype == np.int8
    for g in range(d["G"]):
        counts = np.bincount(h[g], minlength=d["Jc"])
        assert counts.tolist() == [c] * d["Jc"]
    assert set(np.unique(s).tolist()) <= {-1, 1}


def test_plan_deterministic_and_seed_dependent():
    a = oracle.plan(11, 512, 128, 2, 16, 32)
    b = oracle.plan(11, 512, 128, 2, 16, 32)
    c = oracle.plan(12, 512, 128, 2, 16, 32)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert not np.array_equal(a[0], c[0])
    # groups draw different hashes from one stream
    assert not np.array_equal(a[0][0], a[0][1])


def test_plan_shuffle_reaches_every_pairing_uniformly():
    # J = 4 chunks, c = 2: the shuffle has 24 orders mapping onto 3 pairings of
    # the chunks ({01,23}, {02,13}, {03,12}), each hit by 8 orders.  A shuffle
    # that only reaches cyclic orders (a swap range of i instead of i+1) or is
    # otherwise biased shows up as a skewed count.
    counts = {}
    orders = set()
    n = 3000
    for seed in range(n):
        h, s = oracle.plan(seed, 4, 1, 2, 1, 1)
        orders.add(tuple(h[0].tolist()))
        key = frozenset(frozenset(np.flatnonzero(h[0] == t).tolist()) for t in range(2))
        counts[key] = counts.get(key, 0) + 1
    assert len(counts) == 3
    for v in counts.values():
        assert abs(v - n / 3) < 5 * np.sqrt(n * (1 / 3) * (2 / 3))
    # all 6 assignments of chunks to compressed slots 0/1 appear
    assert len(orders) == 6


def test_plan_signs_fair():
    _, s = oracle.plan(5, 4096, 256, 2, 1, 1)
    frac = float(np.mean(s == -1))
    assert abs(frac - 0.5) < 0.01


def test_identity_plan():
    h, s = oracle.identity_plan(64, 8, 8, 4)
    assert (h == np.arange(8)).all() and (s == 1).all()
    oracle.check_plan(h, s, 64, 8, 1, 8, 4)


@pytest.mark.parametrize("K,N,c,BK,BN", SHAPES)
def test_plan_index_partitions_chunks(K, N, c, BK, BN):
    h, s = oracle.plan(3, K, N, c, BK, BN)
    idx, isign = oracle.plan_index(h, s, K, N, c, BK, BN)
    d = oracle.dims(K, N, c, BK, BN)
    for g in range(d["G"]):
        flat = idx[g].reshape(-1)
        assert sorted(flat.tolist()) == list(range(d["J"]))
        for t in range(d["Jc"]):
            assert list(idx[g, t]) == sorted(idx[g, t])
            for r in range(c):
                j = idx[g, t, r]
                assert h[g, j] == t and isign[g, t, r] == s[g, j]


def test_check_plan_rejects_bad_plans():
    K, N, c, BK, BN = 64, 8, 2, 8, 4
    h, s = oracle.plan(1, K, N, c, BK, BN)
    bad = h.copy(); bad[0, 0] = 4  # out of range (Jc = 4)
    with pytest.raises(ValueError):
        oracle.check_plan(bad, s, K, N, c, BK, BN)
    bad = h.copy(); bad[1, 0] = bad[1, 1] if bad[1, 0] != bad[1, 1] else (bad[1, 1] + 1) % 4
    with pytest.raises(ValueError):
        oracle.plan_index(bad, s, K, N, c, BK, BN)  # unbalanced
    oracle.check_plan(bad, s, K, N, c, BK, BN, balanced=False)
    bs = s.copy(); bs[0, 3] = 0
    with pytest.raises(ValueError):
        oracle.check_plan(h, bs, K, N, c, BK, BN)
    with pytest.raises(ValueError):
        oracle.dims(60, 8, 2, 8, 4)  # K % BK
    with pytest.raises(ValueError):
        oracle.dims(48, 8, 4, 8, 4)  # J % c
    with pytest.raises(ValueError):
        oracle.dims(64, 10, 2, 8, 4)  # N % BN


# -------------------------------------------------------------- forward pins
def _brute_dense(Wc, h, s, K, N, BK, BN):
    """Equivalent dense weight written out element by element from the
    parameter-sharing view: weight (n, k) of neuron n is the compressed weight
    its group's hash points at, times the chunk's sign."""
    W = [[0.0] * K for _ in range(N)]
    for n in range(N):
        g = n // BN
        for k in range(K):
            j, u = divmod(k, BK)
            W[n][k] = float(s[g][j]) * float(Wc[n][h[g][j] * BK + u])
    return W


def _naive_matmul_nt(x, W):
    M, N = len(x), len(W)
    K = len(W[0]) if N else 0
    return [[sum(x[m][k] * W[n][k] for k in range(K)) for n in range(N)] for m in range(M)]


TINY = [  # M, K, N, c, BK, BN
    (3, 16, 8, 2, 4, 4),
    (5, 24, 6, 3, 2, 3),
    (1, 32, 8, 4, 2, 2),
    (4, 12, 4, 1, 3, 4),
    (2, 64, 12, 8, 1, 12),
    (0, 16, 8, 2, 4, 4),
]


@pytest.mark.parametrize("M,K,N,c,BK,BN", TINY)
def test_forward_equals_brute_force_dense_integer_exact(M, K, N, c, BK, BN):
    Kc = K // c
    x = draw("int4", 100 + M, (M, K)).astype(np.float64)
    Wc = draw("int4", 200 + K, (N, Kc)).astype(np.float64)
    h, s = oracle.plan(9, K, N, c, BK, BN)
    y = oracle.forward(x, Wc, h, s, K, N, c, BK, BN)
    W = _brute_dense(Wc, h, s, K, N, BK, BN)
    ref = np.array(_naive_matmul_nt(x.tolist(), W), dtype=np.float64).reshape(M, N)
    assert y.shape == (M, N)
    assert np.array_equal(y, ref)  # integers: exact in float64
    assert np.array_equal(oracle.dense_expand(Wc, h, s, K, N, c, BK, BN), np.array(W))


@pytest.mark.parametrize("M,K,N,c,BK,BN", TINY[:5])
def test_forward_equals_brute_force_dense_random(M, K, N, c, BK, BN):
    Kc = K // c
    x = draw("normal", 300 + M, (M, K)).astype(np.float64)
    Wc = draw("normal", 400 + K, (N, Kc)).astype(np.float64)
    h, s = oracle.plan(21, K, N, c, BK, BN)
    y = oracle.forward(x, Wc, h, s, K, N, c, BK, BN)
    ref = np.array(_naive_matmul_nt(x.tolist(), _brute_dense(Wc, h, s, K, N, BK, BN)))
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_identity_plan_is_dense_linear():
    # the tiny float32 workload's shape with c = 1 and the identity plan
    M, K, N, BK, BN = 64, 256, 256, 32, 32
    x = draw("normal", 1, (M, K)).astype(np.float64)
    W = draw("uniform16", 2, (N, K)).astype(np.float64)
    h, s = oracle.identity_plan(K, N, BK, BN)
    y = oracle.forward(x, W, h, s, K, N, 1, BK, BN)
    assert np.allclose(y, x @ W.T, rtol=1e-13, atol=1e-13)
    xi = draw("int4", 3, (M, K)).astype(np.float64)
    Wi = draw("int4", 4, (N, K)).astype(np.float64)
    assert np.array_equal(oracle.forward(xi, Wi, h, s, K, N, 1, BK, BN), xi @ Wi.T)


def test_c1_random_plan_is_signed_chunk_permutation():
    M, K, N, BK, BN = 5, 32, 8, 4, 4
    x = draw("int4", 5, (M, K)).astype(np.float64)
    Wc = draw("int4", 6, (N, K)).astype(np.float64)
    h, s = oracle.plan(2, K, N, 1, BK, BN)
    y = oracle.forward(x, Wc, h, s, K, N, 1, BK, BN)
    for g in range(N // BN):
        # build the permuted, signed input for this group by moving whole chunks
        xp = np.zeros_like(x)
        for j in range(K // BK):
            xp[:, h[g, j] * BK:(h[g, j] + 1) * BK] = s[g, j] * x[:, j * BK:(j + 1) * BK]
        assert np.array_equal(y[:, g * BN:(g + 1) * BN], xp @ Wc[g * BN:(g + 1) * BN].T)


@pytest.mark.parametrize("K,N,c,BK,BN", SHAPES)
def test_sketch_kronecker_form(K, N, c, BK, BN):
    d = oracle.dims(K, N, c, BK, BN)
    M = 3
    x = draw("normal", 7, (M, K)).astype(np.float64)
    h, s = oracle.plan(4, K, N, c, BK, BN)
    z = oracle.sketch(x, h, s, K, N, c, BK, BN)
    for g in range(d["G"]):
        S = np.zeros((d["Jc"], d["J"]))
        S[h[g], np.arange(d["J"])] = s[g]
        # a CountSketch matrix: one nonzero per column, c per row (balanced)
        assert ((S != 0).sum(axis=0) == 1).all() and ((S != 0).sum(axis=1) == c).all()
        P = np.kron(S, np.eye(BK))
        assert np.allclose(z[g], x @ P.T, rtol=1e-13, atol=1e-13)


def test_bk1_bn1_is_textbook_countsketch():
    # BK = 1, BN = 1: every neuron holds its own CountSketch of the input
    # (bucket = hash, random sign), the scatter-add form of the textbook sketch.
    M, K, N, c = 4, 40, 6, 5
    x = draw("normal", 8, (M, K)).astype(np.float64)
    Wc = draw("normal", 9, (N, K // c)).astype(np.float64)
    h, s = oracle.plan(6, K, N, c, 1, 1)
    y = oracle.forward(x, Wc, h, s, K, N, c, 1, 1)
    for n in range(N):
        for m in range(M):
            buckets = np.zeros(K // c)
            np.add.at(buckets, h[n], s[n] * x[m])
            assert abs(y[m, n] - buckets @ Wc[n]) < 1e-12


def test_all_plus_signs_preserve_chunk_sums():
    M, K, N, c, BK, BN = 3, 48, 6, 3, 4, 2
    x = draw("int4", 10, (M, K)).astype(np.float64)
    h, _ = oracle.plan(8, K, N, c, BK, BN)
    s = np.ones_like(h, dtype=np.int8)
    z = oracle.sketch(x, h, s, K, N, c, BK, BN)
    for g in range(N // BN):
        assert np.array_equal(z[g].reshape(M, -1, BK).sum(axis=1), x.reshape(M, -1, BK).sum(axis=1))


def test_group_sign_flip_negates_only_that_group():
    M, K, N, c, BK, BN = 4, 32, 12, 2, 4, 4
    x = draw("normal", 11, (M, K))
    Wc = draw("normal", 12, (N, K // c))
    h, s = oracle.plan(10, K, N, c, BK, BN)
    y = oracle.forward(x, Wc, h, s, K, N, c, BK, BN)
    s2 = s.copy(); s2[1] = -s2[1]
    y2 = oracle.forward(x, Wc, h, s2, K, N, c, BK, BN)
    assert np.array_equal(y2[:, 4:8], -y[:, 4:8])
    assert np.array_equal(y2[:, :4], y[:, :4]) and np.array_equal(y2[:, 8:], y[:, 8:])


def test_linearity():
    M, K, N, c, BK, BN = 5, 32, 8, 4, 2, 4
    h, s = oracle.plan(13, K, N, c, BK, BN)
    x1, x2 = draw("int4", 14, (M, K)), draw("int4", 15, (M, K))
    W1, W2 = draw("int4", 16, (N, K // c)), draw("int4", 17, (N, K // c))
    f = lambda x, W: oracle.forward(x, W, h, s, K, N, c, BK, BN)
    assert np.array_equal(f(2 * x1 - x2, W1), 2 * f(x1, W1) - f(x2, W1))
    assert np.array_equal(f(x1, W1 + 3 * W2), f(x1, W1) + 3 * f(x1, W2))


def test_unbalanced_hash_is_accepted_by_forward():
    M, K, N, c, BK, BN = 2, 16, 4, 2, 2, 4
    x = draw("int4", 18, (M, K)).astype(np.float64)
    Wc = draw("int4", 19, (N, K // c)).astype(np.float64)
    h = np.zeros((1, 8), dtype=np.int32)  # every chunk into slot 0
    s = np.ones((1, 8), dtype=np.int8)
    y = oracle.forward(x, Wc, h, s, K, N, c, BK, BN)
    ref = np.array(_naive_matmul_nt(x.tolist(), _brute_dense(Wc, h, s, K, N, BK, BN)))
    assert np.array_equal(y, ref)


def test_bf16_widening_is_exact():
    vals = np.array([0.0, 1.0, -2.5, 3.140625, 1e-3, -65504.0, 2.0 ** -100], dtype=np.float32)
    bits = f32_to_bf16_bits(vals)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), bf16_bits_to_f32(bits).astype(np.float64))
    assert oracle.bf16_bits_to_f64(np.array([0x3F80, 0xC020], dtype=np.uint16)).tolist() == [1.0, -2.5]


def test_mirror_sketch_rounding():
    # c = 2 with bf16 inputs: float32 holds the pair sum exactly unless the
    # exponents differ a lot, so the mirror sketch's bf16 value must be the
    # ties-to-even rounding of the float32 sum; the bit-level encoder used for
    # inputs is an independent rounding routine to compare with.
    M, K, N, c, BK, BN = 64, 128, 8, 2, 8, 8
    xb = f32_to_bf16_bits(draw("normal", 20, (M, K)))
    x = bf16_bits_to_f32(xb)
    h, s = oracle.plan(14, K, N, c, BK, BN)
    zr = oracle.sketch_rounded(x, h, s, K, N, c, BK, BN, to_bf16=True)
    z32 = oracle.sketch_rounded(x, h, s, K, N, c, BK, BN, to_bf16=False)
    z = oracle.sketch(x.astype(np.float64), h, s, K, N, c, BK, BN)
    assert np.array_equal(z32, z)  # exact pair sums
    ref = bf16_bits_to_f32(f32_to_bf16_bits(z32.astype(np.float32))).astype(np.float64)
    assert np.array_equal(zr, ref)
    # ties go to even
    t = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], dtype=np.float32)
    from oracle.ss1_oracle import _round_f32_to_bf16
    assert _round_f32_to_bf16(t).tolist() == [1.0, 1.0 + 2.0 ** -6]


def test_flops_accounting():
    f = oracle.flops(8192, 768, 3072, 2)
    assert f["dense_equiv"] == 2 * 8192 * 768 * 3072 and f["compressed"] * 2 == f["dense_equiv"]


def test_all_small_pairings_enumerated_match_dense():
    # exhaustive over every balanced plan and sign pattern of a 4-chunk, c = 2
    # layer with one group: forward must equal the dense expansion each time
    M, K, N, c, BK, BN = 2, 8, 2, 2, 2, 2
    x = draw("int4", 21, (M, K)).astype(np.float64)
    Wc = draw("int4", 22, (N, K // c)).astype(np.float64)
    for perm in itertools.permutations(range(4)):
        h = np.array([[p // 2 for p in np.argsort(perm)]], dtype=np.int32)
        for signs in itertools.product((-1, 1), repeat=4):
            s = np.array([signs], dtype=np.int8)
            y = oracle.forward(x, Wc, h, s, K, N, c, BK, BN)
            ref = np.array(_naive_matmul_nt(x.tolist(), _brute_dense(Wc, h, s, K, N, BK, BN)))
            assert np.array_equal(y, ref)


def test_plan_worked_examples():
    with open(os.path.join(GOLDEN, "plan_worked_examples.txt")) as f:
        rows = [l for l in f if l.strip() and not l.startswith("#")]
    assert rows
    for line in rows:
        head, hs, ss = (p.split() for p in line.split("|"))
        seed, K, N, c, BK, BN = (int(v) for v in head)
        h, s = oracle.plan(seed, K, N, c, BK, BN)
        assert h[0].tolist() == [int(v) for v in hs]
        assert s[0, :len(ss)].tolist() == [int(v) for v in ss]


# ----------------------------------------------------------- projection pins
# The projection is pinned against an explicit least-squares solve of the
# expansion matrix (numpy.linalg.lstsq), against dense_expand (left inverse,
# exact on integers), and by orthogonality of its residual.
PROJ_SHAPES = [  # K, N, c, BK, BN
    (64, 8, 2, 8, 4), (96, 12, 4, 8, 6), (48, 6, 1, 8, 3), (72, 8, 3, 4, 8), (256, 16, 8, 8, 16)]


def _expansion_matrix(hash_, sign, g, K, c, BK):
    """[K][Kc] matrix E with dense row = E @ compressed row for group g, built
    entry by entry from the plan's definition."""
    J = K // BK
    Kc = K // c
    E = np.zeros((K, Kc))
    for j in range(J):
        t = int(hash_[g, j])
        for u in range(BK):
            E[j * BK + u, t * BK + u] = float(sign[g, j])
    return E


@pytest.mark.parametrize("K,N,c,BK,BN", PROJ_SHAPES)
def test_project_matches_least_squares_solve(K, N, c, BK, BN):
    h, s = oracle.plan(21, K, N, c, BK, BN)
    W = np.random.default_rng(3).standard_normal((N, K))
    got = oracle.project(W, h, s, K, N, c, BK, BN)
    for n in range(N):
        E = _expansion_matrix(h, s, n // BN, K, c, BK)
        ref = np.linalg.lstsq(E, W[n], rcond=None)[0]
        np.testing.assert_allclose(got[n], ref, rtol=0, atol=1e-12)


def test_project_least_squares_unbalanced_and_empty_chunks():
    K, N, c, BK, BN = 48, 4, 2, 8, 2   # J = 6, Jc = 3
    h, s = oracle.plan(4, K, N, c, BK, BN)
    h = h.copy()
    h[0] = [0, 0, 0, 2, 2, 0]          # chunk 1 of group 0 gets no source, chunk 0 four
    W = np.random.default_rng(5).standard_normal((N, K))
    got = oracle.project(W, h, s, K, N, c, BK, BN)
    for n in range(N):
        E = _expansion_matrix(h, s, n // BN, K, c, BK)
        ref = np.linalg.lstsq(E, W[n], rcond=None)[0]   # minimum-norm: 0 on the empty chunk
        np.testing.assert_allclose(got[n], ref, rtol=0, atol=1e-12)
    assert not got[:BN, BK:2 * BK].any()


@pytest.mark.parametrize("K,N,c,BK,BN", [p for p in PROJ_SHAPES if p[2] in (1, 2, 4, 8)])
def test_project_is_exact_left_inverse_of_dense_expand(K, N, c, BK, BN):
    h, s = oracle.plan(8, K, N, c, BK, BN)
    Wc = np.random.default_rng(6).integers(-4, 5, size=(N, K // c)).astype(np.float64)
    W = oracle.dense_expand(Wc, h, s, K, N, c, BK, BN)
    assert np.array_equal(oracle.project(W, h, s, K, N, c, BK, BN), Wc)


@pytest.mark.parametrize("K,N,c,BK,BN", [p for p in PROJ_SHAPES if p[2] in (1, 2, 4, 8)])
def test_project_residual_is_orthogonal_to_the_sharing_subspace(K, N, c, BK, BN):
    h, s = oracle.plan(9, K, N, c, BK, BN)
    W = np.random.default_rng(7).integers(-8, 9, size=(N, K)).astype(np.float64)
    R = W - oracle.dense_expand(oracle.project(W, h, s, K, N, c, BK, BN), h, s, K, N, c, BK, BN)
    assert not oracle.project(R, h, s, K, N, c, BK, BN).any()      # exact: c is a power of 2
    V = np.random.default_rng(8).standard_normal((N, K // c))
    inner = np.sum(R * oracle.dense_expand(V, h, s, K, N, c, BK, BN))
    assert abs(inner) <= 1e-9 * np.abs(R).sum()


def test_project_c1_inverts_signed_permutation():
    K, N, c, BK, BN = 64, 6, 1, 8, 3
    h, s = oracle.plan(10, K, N, c, BK, BN)
    W = np.random.default_rng(11).standard_normal((N, K))
    Wc = oracle.project(W, h, s, K, N, c, BK, BN)
    assert np.array_equal(oracle.dense_expand(Wc, h, s, K, N, c, BK, BN), W)


def test_project_rounded_mirror():
    K, N, c, BK, BN = 64, 8, 4, 8, 4
    h, s = oracle.plan(12, K, N, c, BK, BN)
    # integer inputs: float32 sums and the division by 4 are exact, and the
    # quarter-integers below 2^6 keep at most 8 significant bits
    W = np.random.default_rng(13).integers(-4, 5, size=(N, K)).astype(np.float64)
    exact = oracle.project(W, h, s, K, N, c, BK, BN)
    for to_bf16 in (False, True):
        assert np.array_equal(oracle.project_rounded(W, h, s, K, N, c, BK, BN, to_bf16), exact)
    # c = 3: the division rounds; the mirror gives the float32 quotient
    K3, c3 = 72, 3
    h3, s3 = oracle.plan(14, K3, N, c3, 4, BN)
    W3 = np.random.default_rng(15).integers(-4, 5, size=(N, K3)).astype(np.float64)
    ex3 = oracle.project(W3, h3, s3, K3, N, c3, 4, BN)
    m3 = oracle.project_rounded(W3, h3, s3, K3, N, c3, 4, BN, False)
    assert np.array_equal(m3, ex3.astype(np.float32).astype(np.float64))


# ------------------------------------------------------------ MLP pair pins
def test_gelu_against_normal_cdf_and_identities():
    from scipy.stats import norm
    v = np.concatenate([np.linspace(-8, 8, 161), [-1e-3, 1e-3, 30.0, -30.0]])
    np.testing.assert_allclose(oracle.gelu(v), v * norm.cdf(v), rtol=1e-12, atol=1e-300)
    # GELU(v) - GELU(-v) = v (Phi(v) + Phi(-v) = 1); GELU(0) = 0
    np.testing.assert_allclose(oracle.gelu(v) - oracle.gelu(-v), v, rtol=1e-14, atol=1e-14)
    assert oracle.gelu(0.0) == 0.0
    assert oracle.gelu(30.0) == 30.0 and abs(oracle.gelu(-30.0)) < 1e-190


def _layer(seed, K, N, c, BK, BN, identity=False, integer=False):
    h, s = oracle.identity_plan(K, N, BK, BN) if identity else oracle.plan(seed, K, N, c, BK, BN)
    g = np.random.default_rng(seed)
    Wc = (g.integers(-2, 3, size=(N, K // c)).astype(np.float64) if integer
          else g.standard_normal((N, K // c)) * 0.05)
    return {"Wc": Wc, "hash": h, "sign": s, "K": K, "N": N, "c": c, "BK": BK, "BN": BN}


def test_mlp_identity_plans_equal_dense_mlp():
    from scipy.stats import norm
    up = _layer(1, 64, 96, 1, 8, 16, identity=True)
    down = _layer(2, 96, 32, 1, 8, 16, identity=True)
    x = np.random.default_rng(3).standard_normal((7, 64))
    a = x @ up["Wc"].T
    y_ref = (a * norm.cdf(a)) @ down["Wc"].T
    h, y = oracle.mlp_forward(x, up, down)
    np.testing.assert_allclose(y, y_ref, rtol=1e-12, atol=1e-12)


def test_mlp_equals_dense_expansions():
    from scipy.stats import norm
    up = _layer(4, 128, 64, 2, 16, 16)
    down = _layer(5, 64, 48, 4, 8, 16)
    x = np.random.default_rng(6).standard_normal((5, 128))
    Wu = oracle.dense_expand(up["Wc"], up["hash"], up["sign"], 128, 64, 2, 16, 16)
    Wd = oracle.dense_expand(down["Wc"], down["hash"], down["sign"], 64, 48, 4, 8, 16)
    a = x @ Wu.T
    h, y = oracle.mlp_forward(x, up, down)
    np.testing.assert_allclose(h, a * norm.cdf(a), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(y, (a * norm.cdf(a)) @ Wd.T, rtol=1e-11, atol=1e-12)
    with pytest.raises(ValueError):
        oracle.mlp_forward(x, up, _layer(7, 32, 48, 2, 8, 16))


def test_mlp_rounded_h_is_bf16():
    up = _layer(8, 64, 32, 2, 8, 16)
    down = _layer(9, 32, 16, 2, 8, 16)
    x = np.random.default_rng(10).standard_normal((4, 64))
    h, y = oracle.mlp_forward(x, up, down, round_h_to_bf16=True)
    bits = f32_to_bf16_bits(h.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f32(bits).astype(np.float64), h)
    h0, _ = oracle.mlp_forward(x, up, down)
    assert np.all(np.abs(h - h0) <= 2.0 ** -8 * np.abs(h0))


# ---------------------------------------------------------------- fp8 pins
# The E4M3 codec is pinned against torch's float8_e4m3fn (an independent
# implementation of the same OCP format) on every code and on random values,
# and on exact midpoints (ties to even) and saturation.
def test_e4m3_decode_matches_torch_on_every_code():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))
    assert np.nanmax(got) == oracle.E4M3_MAX and got[1] == 2.0 ** -9


def test_e4m3_encode_matches_torch_and_rounds_ties_to_even():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(20)
    v = np.concatenate([g.standard_normal(4000) * 50, g.standard_normal(2000) * 0.01,
                        g.uniform(-448, 448, 2000), [0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10]])
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(v.astype(np.float32).astype(np.float64)), ref)
    # every midpoint between neighbouring finite positive codes goes to the even code
    vals = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    codes = oracle.e4m3_encode(mids)
    lo = np.arange(0, 0x7E)
    assert np.array_equal(codes, np.where(lo % 2 == 0, lo, lo + 1))
    # saturation instead of NaN past the largest finite value
    assert list(oracle.e4m3_encode([1000.0, -1e9, 464.0])) == [0x7E, 0xFE, 0x7E]


def test_quantize_fp8_rows():
    g = np.random.default_rng(21)
    W = (g.standard_normal((6, 96)) * 0.02).astype(np.float32)
    W[3] = 0.0
    codes, scale = oracle.quantize_fp8_rows(W)
    assert scale.dtype == np.float32 and scale[3] == 1.0 and not codes[3].any()
    deq = oracle.dequantize_fp8_rows(codes, scale)
    for n in (0, 1, 2, 4, 5):
        assert scale[n] == np.float32(np.max(np.abs(W[n])) / np.float32(448.0))
        assert np.max(np.abs(oracle.e4m3_decode(codes[n]))) == 448.0      # the row maximum maps to 448
        # nearest-code error: half a quantum, at most 2^-4 of the value for normals
        q = W[n].astype(np.float64) / scale[n]
        err = np.abs(oracle.e4m3_decode(codes[n]) - q)
        assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(q), 2.0 ** -10) + 1e-12)
    np.testing.assert_allclose(deq[0], W[0], rtol=2 ** -4, atol=scale[0] * 2.0 ** -10)


# ----------------------------------------------------------- backward pins
BWD_SHAPES = [(5, 64, 8, 2, 8, 4), (3, 96, 12, 4, 8, 6), (4, 48, 6, 1, 8, 3), (6, 72, 8, 3, 4, 8)]


@pytest.mark.parametrize("M,K,N,c,BK,BN", BWD_SHAPES)
def test_backward_adjoint_identities_integer_exact(M, K, N, c, BK, BN):
    """y is linear in x and in Wc: <dy, y> = <dx, x> = <dWc, Wc>, exactly on
    integer inputs in float64."""
    g = np.random.default_rng(M * K)
    h, s = oracle.plan(33, K, N, c, BK, BN)
    x = g.integers(-4, 5, (M, K)).astype(np.float64)
    Wc = g.integers(-4, 5, (N, K // c)).astype(np.float64)
    dy = g.integers(-4, 5, (M, N)).astype(np.float64)
    y = oracle.forward(x, Wc, h, s, K, N, c, BK, BN)
    dx, dWc = oracle.backward(x, Wc, dy, h, s, K, N, c, BK, BN)
    assert np.sum(dy * y) == np.sum(dx * x) == np.sum(dWc * Wc)


@pytest.mark.parametrize("M,K,N,c,BK,BN", BWD_SHAPES)
def test_backward_dx_equals_dense_expansion(M, K, N, c, BK, BN):
    g = np.random.default_rng(K)
    h, s = oracle.plan(34, K, N, c, BK, BN)
    x = g.standard_normal((M, K))
    Wc = g.standard_normal((N, K // c))
    dy = g.standard_normal((M, N))
    dx, _ = oracle.backward(x, Wc, dy, h, s, K, N, c, BK, BN)
    np.testing.assert_allclose(dx, dy @ oracle.dense_expand(Wc, h, s, K, N, c, BK, BN), rtol=1e-12, atol=1e-12)


def test_backward_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    M, K, N, c, BK, BN = 7, 128, 32, 4, 8, 8
    h, s = oracle.plan(35, K, N, c, BK, BN)
    g = np.random.default_rng(36)
    x = g.standard_normal((M, K))
    Wc = g.standard_normal((N, K // c))
    dy = g.standard_normal((M, N))
    # dense weight built from Wc by torch indexing: W[n, j*BK+u] = sign * Wc[n, hash*BK+u]
    J = K // BK
    col = np.empty((N, K), dtype=np.int64)
    sg = np.empty((N, K))
    for n in range(N):
        for j in range(J):
            col[n, j * BK:(j + 1) * BK] = h[n // BN, j] * BK + np.arange(BK)
            sg[n, j * BK:(j + 1) * BK] = s[n // BN, j]
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(Wc, requires_grad=True)
    W = torch.gather(wt, 1, torch.tensor(col)) * torch.tensor(sg)
    (xt @ W.T).backward(torch.tensor(dy))
    dx, dWc = oracle.backward(x, Wc, dy, h, s, K, N, c, BK, BN)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dWc, wt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_backward_dw_mirror_rounds_only_the_sketch():
    M, K, N, c, BK, BN = 6, 64, 8, 2, 8, 4
    h, s = oracle.plan(37, K, N, c, BK, BN)
    g = np.random.default_rng(38)
    x = g.integers(-4, 5, (M, K)).astype(np.float64)     # integer sketch: exact in bf16
    dy = g.standard_normal((M, N))
    Wc = np.zeros((N, K // c))
    _, dWc = oracle.backward(x, Wc, dy, h, s, K, N, c, BK, BN)
    assert np.array_equal(oracle.backward_dw_mirror(x, dy, h, s, K, N, c, BK, BN), dWc)


# --------------------------------------------------- pins of forward_mirror
# forward_mirror is the elementwise bar of the device parity tests for the
# kernels that round the sketch to bf16, so it is pinned here against code
# that shares nothing with it: torch CPU matmuls of the Kronecker (CountSketch
# matrix) form, and torch's own float32 -> bf16 conversion (nearest, ties to
# even) in place of the oracle's frexp/ldexp rounding.

def _torch_mirror(x32, Wc, h, s, K, N, c, BK, BN, group_shift=0):
    """y from the bf16-rounded float32 sketch, built with torch: z_g is x times
    the transposed Kronecker matrix (S_g kron I_BK) in float32 -- for c = 2
    every output sums exactly two signed inputs, so any summation order gives
    the one rounding of that pair -- then rounded by torch's bf16 conversion
    and contracted in float64.  ``group_shift`` pairs group g's sketch with
    group g + shift's weight rows (a planted slip)."""
    torch = pytest.importorskip("torch")
    d = oracle.dims(K, N, c, BK, BN)
    J, Jc, G = d["J"], d["Jc"], d["G"]
    xt = torch.from_numpy(np.asarray(x32, dtype=np.float32))
    W = torch.from_numpy(np.asarray(Wc, dtype=np.float64))
    y = torch.empty((xt.shape[0], N), dtype=torch.float64)
    eye = torch.eye(BK, dtype=torch.float32)
    for g in range(G):
        S = torch.zeros((Jc, J), dtype=torch.float32)
        S[torch.from_numpy(h[g].astype(np.int64)), torch.arange(J)] = torch.from_numpy(s[g].astype(np.float32))
        z = (xt @ torch.kron(S, eye).T).to(torch.bfloat16).to(torch.float64)
        gw = (g + group_shift) % G
        y[:, g * BN:(g + 1) * BN] = z @ W[gw * BN:(gw + 1) * BN].T
    return y.numpy()


def test_forward_mirror_integer_inputs_equal_forward_bit_exact():
    # integer inputs in {-4..4}: each sketch value is an integer of magnitude
    # at most 4c, exact in bf16, so the rounded mirror is the definition itself
    for K, N, c, BK, BN in [(256, 64, 2, 32, 32), (384, 48, 3, 16, 16), (512, 32, 4, 64, 8)]:
        h, s = oracle.plan(41 + c, K, N, c, BK, BN)
        g = np.random.default_rng(42 + c)
        x = g.integers(-4, 5, (9, K)).astype(np.float64)
        Wc = g.integers(-4, 5, (N, K // c)).astype(np.float64)
        ref = oracle.forward(x, Wc, h, s, K, N, c, BK, BN)
        for rounded in (True, False):
            assert np.array_equal(oracle.forward_mirror(x, Wc, h, s, K, N, c, BK, BN, rounded), ref)


def test_forward_mirror_c2_matches_torch_kronecker_form():
    M, K, N, c, BK, BN = 33, 512, 96, 2, 32, 32
    h, s = oracle.plan(43, K, N, c, BK, BN)
    x = bf16_bits_to_f32(f32_to_bf16_bits(draw("normal", 44, (M, K))))
    Wc = bf16_bits_to_f32(f32_to_bf16_bits(draw("normal002", 45, (N, K // c)))).astype(np.float64)
    mir = oracle.forward_mirror(x, Wc, h, s, K, N, c, BK, BN, True)
    ref = _torch_mirror(x, Wc, h, s, K, N, c, BK, BN)
    scale = np.max(np.abs(ref))
    assert np.max(np.abs(mir - ref)) <= 1e-12 * scale
    # the rounding of the sketch is visible at this size: the unrounded mirror
    # and the exact forward differ from the rounded one by far more than 1e-12
    unr = oracle.forward_mirror(x, Wc, h, s, K, N, c, BK, BN, False)
    assert np.max(np.abs(unr - ref)) > 1e-6 * scale
    assert np.array_equal(unr, oracle.forward(x, Wc, h, s, K, N, c, BK, BN))  # exact pair sums


def test_forward_mirror_pin_catches_a_wrong_group():
    # a planted slip on the reference side (group g's sketch against group
    # g+1's weight rows) must fail the same 1e-12 comparison by a wide margin
    M, K, N, c, BK, BN = 17, 256, 64, 2, 32, 32
    h, s = oracle.plan(46, K, N, c, BK, BN)
    x = bf16_bits_to_f32(f32_to_bf16_bits(draw("normal", 47, (M, K))))
    Wc = draw("normal002", 48, (N, K // c)).astype(np.float64)
    mir = oracle.forward_mirror(x, Wc, h, s, K, N, c, BK, BN, True)
    bad = _torch_mirror(x, Wc, h, s, K, N, c, BK, BN, group_shift=1)
    assert np.max(np.abs(mir - bad)) > 1e-2 * np.max(np.abs(mir))


def test_forward_mirror_c4_ascending_float32_sum():
    # c = 4: the float32 sum depends on the order; the mirror adds the
    # sources of each compressed chunk in ascending chunk order.  Rebuilt here
    # from the inverse index with torch float32 adds and torch's bf16 rounding.
    torch = pytest.importorskip("torch")
    M, K, N, c, BK, BN = 11, 1024, 32, 4, 32, 16
    h, s = oracle.plan(49, K, N, c, BK, BN)
    idx, isg = oracle.plan_index(h, s, K, N, c, BK, BN)
    d = oracle.dims(K, N, c, BK, BN)
    x = bf16_bits_to_f32(f32_to_bf16_bits(draw("normal", 50, (M, K))))
    Wc = draw("normal002", 51, (N, K // c)).astype(np.float64)
    xt = torch.from_numpy(x)
    ref = np.empty((M, N))
    for g in range(d["G"]):
        parts = []
        for t in range(d["Jc"]):
            acc = None
            for r in range(c):
                j = int(idx[g, t, r])
                assert r == 0 or j > int(idx[g, t, r - 1])
                term = float(isg[g, t, r]) * xt[:, j * BK:(j + 1) * BK]
                acc = term if acc is None else acc + term
            parts.append(acc.to(torch.bfloat16).to(torch.float64))
        z = torch.cat(parts, dim=1).numpy()
        ref[:, g * BN:(g + 1) * BN] = z @ Wc[g * BN:(g + 1) * BN].T
    mir = oracle.forward_mirror(x, Wc, h, s, K, N, c, BK, BN, True)
    assert np.max(np.abs(mir - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_forward_float32_steps_match_float64():
    # the float32 run of the same steps (the benchmark's CPU-speed baseline)
    # agrees with the float64 definition to float32 accuracy, and the default
    # stays float64
    M, K, N, c, BK, BN = 40, 512, 96, 2, 32, 32
    h, s = oracle.plan(52, K, N, c, BK, BN)
    x = draw("normal", 53, (M, K)).astype(np.float64)
    Wc = draw("normal002", 54, (N, K // c)).astype(np.float64)
    y64 = oracle.forward(x, Wc, h, s, K, N, c, BK, BN)
    y32 = oracle.forward(x, Wc, h, s, K, N, c, BK, BN, dtype=np.float32)
    assert y64.dtype == np.float64 and y32.dtype == np.float32
    assert np.max(np.abs(y32 - y64)) <= 1e-5 * np.max(np.abs(y64))
