"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's own formulas: each checks it against a
hand-worked value, exact rational arithmetic of the definition, a different
formulation of the same quantity (the quadratic "attention" form of Mamba-2,
the chunked WY form of the delta rule), or a case in which the sketch read must
be exact.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import BatchOracle, ItemOracle, plan, transition
from workloads import CONFIGS, Workload

KINDS = ("mamba2", "gdn", "kda")


# ---------------------------------------------------------------------------
# hand-worked fixtures
# ---------------------------------------------------------------------------
def test_tiny_hand_cases(golden_dir):
    with open(os.path.join(golden_dir, "tiny_hand.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        kind = case["kind"]
        S = np.array(case["S_init"])
        om = np.array([[1.0, 0.0]])
        sk = ItemOracle(kind, 2, S, om, om)
        dn = ItemOracle(kind, 2, S)
        for t, tok in enumerate(case["tokens"]):
            y, ye = sk.read(tok["q"], tok["k"], tok["v"], tok["a"], tok.get("beta"))
            yd, _ = dn.read(tok["q"], tok["k"], tok["v"], tok["a"], tok.get("beta"))
            assert y[0] == pytest.approx(case["y_sketch"][t], abs=1e-12), (kind, t)
            assert ye[0] == pytest.approx(case["y_exact"][t], abs=1e-12), (kind, t)
            assert yd[0] == pytest.approx(case["y_exact"][t], abs=1e-12), (kind, t)
            if sk.j == 2:
                sk.flush()
                dn.flush()
                np.testing.assert_allclose(sk.S0, case["S_after_flush"], atol=1e-12)
                np.testing.assert_allclose(sk.Z, case["Z_after_flush"], atol=1e-12)


def test_plan_hand_example(golden_dir):
    with open(os.path.join(golden_dir, "plan_small.json")) as f:
        g = json.load(f)
    p = plan(g["rank"], g["group"], g["G"], g["K"], g["basis_rows"], g["rank_cap"])
    assert [list(x) for x in p["frames"]] == g["frames"]
    for key in ("frame_index", "frame_row_off", "z_row_off", "bucket", "order"):
        assert p[key].tolist() == g[key], key


def test_plan_properties_random():
    rng = np.random.default_rng(7)
    for _ in range(200):
        H = int(rng.integers(1, 140))
        G = int(rng.integers(1, 9))
        rank = rng.integers(0, 50, size=H)
        rank[rng.random(H) < 0.2] = 0
        group = rng.integers(0, G, size=H)
        p = plan(rank, group, G, 128, 79, 49)
        fr = p["frames"]
        assert fr == sorted(set(fr))
        assert p["order"].tolist() != [] or H == 0
        assert sorted(p["order"].tolist()) == list(range(H))
        for h in range(H):
            if rank[h] == 0:
                assert p["frame_index"][h] == -1 and p["bucket"][h] == 0
            else:
                assert fr[p["frame_index"][h]] == (group[h], rank[h])
                assert 1 <= p["bucket"][h] <= 7
                assert (rank[h] - 1) // 8 + 1 == p["bucket"][h]
        assert np.all(np.diff(p["z_row_off"]) == rank)
        assert np.all(np.diff(p["frame_row_off"]) == [r for _, r in fr])
        keys = [(p["bucket"][h] != 0, -p["bucket"][h], h) for h in p["order"]]
        assert keys == sorted(keys)


def test_plan_rejects_bad_tables():
    with pytest.raises(ValueError):
        plan([50], [0], 1, 128, 79, 49)
    with pytest.raises(ValueError):
        plan([-1], [0], 1, 128, 79, 49)
    with pytest.raises(ValueError):
        plan([3], [1], 1, 128, 79, 49)


# ---------------------------------------------------------------------------
# exact rational brute force on tiny inputs
# ---------------------------------------------------------------------------
def _fr_matmul(A, B):
    return [[sum(A[i][t] * B[t][j] for t in range(len(B))) for j in range(len(B[0]))]
            for i in range(len(A))]


def _fr_T(A):
    return [list(r) for r in zip(*A)]


def _fr_eye(n):
    return [[Fraction(int(i == j)) for j in range(n)] for i in range(n)]


def _fr_transition(kind, a, beta, k):
    K = len(k)
    E = [[Fraction(int(i == j)) - beta * k[i] * k[j] for j in range(K)] for i in range(K)]
    if kind == "mamba2":
        return [[a * Fraction(int(i == j)) for j in range(K)] for i in range(K)]
    if kind == "gdn":
        return [[a * E[i][j] for j in range(K)] for i in range(K)]
    return [[E[i][j] * a[j] for j in range(K)] for i in range(K)]


def _fr_pinvT(Om):
    """pinv(Omega)^T = (Omega Omega^T)^-1 Omega for full-row-rank Omega (r <= 2)."""
    G = _fr_matmul(Om, _fr_T(Om))
    if len(G) == 1:
        inv = [[1 / G[0][0]]]
    else:
        det = G[0][0] * G[1][1] - G[0][1] * G[1][0]
        inv = [[G[1][1] / det, -G[0][1] / det], [-G[1][0] / det, G[0][0] / det]]
    return _fr_matmul(inv, Om)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("r", [1, 2])
def test_fraction_brute_force(kind, r):
    """Exact arithmetic of the definition: the sketch output equals the exact
    output minus S_0^T (I - Omega_r^T F_r) q~, with F_r = pinv(Omega_r)^T formed
    exactly; the oracle (fp64) must agree to 1e-12 in both modes."""
    rng = np.random.default_rng(100 + r + 10 * KINDS.index(kind))
    K, V, W, T = 3, 2, 2, 5

    def rat():
        return Fraction(int(rng.integers(-9, 10)), int(rng.integers(1, 7)))

    S = [[rat() for _ in range(V)] for _ in range(K)]
    Om = [[rat() for _ in range(K)] for _ in range(r)]
    while True:  # full row rank
        Gm = _fr_matmul(Om, _fr_T(Om))
        det = Gm[0][0] if r == 1 else Gm[0][0] * Gm[1][1] - Gm[0][1] * Gm[1][0]
        if det != 0:
            break
        Om = [[rat() for _ in range(K)] for _ in range(r)]
    F = _fr_pinvT(Om)
    toks = []
    for _ in range(T):
        k = [rat() for _ in range(K)]
        a = [Fraction(int(rng.integers(1, 5)), 4) for _ in range(K)] if kind == "kda" \
            else Fraction(int(rng.integers(1, 5)), 4)
        toks.append(dict(q=[rat() for _ in range(K)], k=k, v=[rat() for _ in range(V)],
                         a=a, beta=Fraction(int(rng.integers(0, 4)), 3)))

    # exact trajectory
    S_init = [row[:] for row in S]
    S0 = [row[:] for row in S]
    P = _fr_eye(K)
    ImOF = [[Fraction(int(i == j)) - sum(Om[m][i] * F[m][j] for m in range(r)) for j in range(K)]
            for i in range(K)]
    want_sk, want_ex = [], []
    j = 0
    for tok in toks:
        beta = Fraction(1) if kind == "mamba2" else tok["beta"]
        M = _fr_transition(kind, tok["a"], beta, tok["k"])
        S = _fr_matmul(M, S)
        S = [[S[i][c] + beta * tok["k"][i] * tok["v"][c] for c in range(V)] for i in range(K)]
        P = _fr_matmul(M, P)
        j += 1
        y = [sum(S[i][c] * tok["q"][i] for i in range(K)) for c in range(V)]
        qt = [sum(P[i][m] * tok["q"][i] for i in range(K)) for m in range(K)]
        corr = [sum(ImOF[i][m] * qt[m] for m in range(K)) for i in range(K)]
        err = [-sum(S0[i][c] * corr[i] for i in range(K)) for c in range(V)]
        want_ex.append([float(x) for x in y])
        want_sk.append([float(y[c] + err[c]) for c in range(V)])
        if j == W:
            S0 = [row[:] for row in S]
            P = _fr_eye(K)
            j = 0

    f = lambda A: np.array([[float(x) for x in row] for row in A])  # noqa: E731
    item = ItemOracle(kind, W, f(S_init), f(Om), f(F))
    batch = BatchOracle(kind, W, f(S_init)[None], [f(Om)], [f(F)])
    for t, tok in enumerate(toks):
        args = [np.array([float(x) for x in tok["q"]]), np.array([float(x) for x in tok["k"]]),
                np.array([float(x) for x in tok["v"]]),
                (np.array([float(x) for x in tok["a"]]) if kind == "kda" else float(tok["a"])),
                float(tok["beta"])]
        y1, y1e = item.read(*args)
        yb, ybe = batch.read(args[0][None], args[1][None], args[2][None],
                             np.atleast_1d(np.asarray(args[3]))[None] if kind == "kda"
                             else np.array([args[3]]), np.array([args[4]]))
        np.testing.assert_allclose(y1, want_sk[t], rtol=0, atol=1e-12)
        np.testing.assert_allclose(y1e, want_ex[t], rtol=0, atol=1e-12)
        np.testing.assert_allclose(yb[0], want_sk[t], rtol=0, atol=1e-12)
        np.testing.assert_allclose(ybe[0], want_ex[t], rtol=0, atol=1e-12)
        if item.j == W:
            item.flush()
            batch.flush()


# ---------------------------------------------------------------------------
# cases where the sketch read is exact
# ---------------------------------------------------------------------------
def _random_tokens(rng, kind, K, V, T, beta=None, a_uniform=False):
    toks = []
    for _ in range(T):
        k = rng.standard_normal(K)
        k /= np.linalg.norm(k)
        if kind == "kda":
            a = np.full(K, rng.uniform(0.6, 1.0)) if a_uniform else rng.uniform(0.6, 1.0, K)
        else:
            a = rng.uniform(0.6, 1.0)
        toks.append(dict(q=rng.standard_normal(K), k=k, v=rng.standard_normal(V), a=a,
                         beta=(rng.uniform(0.1, 0.9) if beta is None else beta)))
    return toks


@pytest.mark.parametrize("kind", KINDS)
def test_full_orthonormal_basis_reads_exactly(kind):
    """r = K with an orthonormal K x K basis and F = Omega: the sketch holds the
    whole state, so the sketch read equals the full read."""
    rng = np.random.default_rng(1)
    K, V, W = 16, 5, 4
    Om, _ = np.linalg.qr(rng.standard_normal((K, K)))
    Om = Om.T
    S = rng.standard_normal((K, V))
    o = ItemOracle(kind, W, S, Om, Om)
    for tok in _random_tokens(rng, kind, K, V, 3 * W + 1):
        y, ye = o.read(tok["q"], tok["k"], tok["v"], tok["a"], tok["beta"])
        np.testing.assert_allclose(y, ye, rtol=0, atol=1e-12)
        if o.j == W:
            o.flush()


def test_mamba2_query_in_span_reads_exactly():
    """Mamba-2 with no query noise: q~ = (product of decays) q stays in the span
    of Omega_r, so Z^T F_r q~ = S_0^T q~ and the sketch read is exact."""
    cfg = CONFIGS["c0"]
    wl = Workload(cfg)
    rng = np.random.default_rng(2)
    r = 6
    Om = wl.basis[0, :r].astype(np.float64)
    F = wl.fmap(0, r).astype(np.float64)
    S = wl.state_item(0, 0)
    o = ItemOracle("mamba2", 16, S, Om, F)
    for tok in _random_tokens(rng, "mamba2", 128, 80, 40):
        q = rng.standard_normal(r) @ Om
        y, ye = o.read(q, tok["k"], tok["v"], tok["a"])
        # F is the float32 stored map: exact up to its rounding
        np.testing.assert_allclose(y, ye, rtol=0, atol=1e-5 * np.abs(ye).max())
        if o.j == 16:
            o.flush()


@pytest.mark.parametrize("kind", KINDS)
def test_sketch_error_closed_form(kind):
    """y^ - y = -S_0^T (I - Omega_r^T F_r) q~ at every window position."""
    rng = np.random.default_rng(3)
    K, V, W, r = 12, 4, 5, 3
    Om = rng.standard_normal((r, K))
    F = np.linalg.pinv(Om).T
    S = rng.standard_normal((K, V))
    o = ItemOracle(kind, W, S, Om, F)
    S0 = S.copy()
    P = np.eye(K)
    for tok in _random_tokens(rng, kind, K, V, 2 * W + 2):
        M = transition(kind, tok["a"], tok["beta"], tok["k"])
        P = M @ P
        y, ye = o.read(tok["q"], tok["k"], tok["v"], tok["a"], tok["beta"])
        qt = P.T @ tok["q"]
        want = ye - S0.T @ ((np.eye(K) - Om.T @ F) @ qt)
        np.testing.assert_allclose(y, want, rtol=0, atol=1e-11)
        if o.j == W:
            o.flush()
            S0 = o.S0.copy()
            P = np.eye(K)


# ---------------------------------------------------------------------------
# other formulations of the exact recurrence
# ---------------------------------------------------------------------------
def test_mamba2_matches_quadratic_attention_form():
    """Mamba-2's dual form: y_t = (prod_{l<=t} a_l) S_init^T q_t
    + sum_{i<=t} (prod_{i<l<=t} a_l) (k_i . q_t) v_i; flushes change nothing."""
    rng = np.random.default_rng(4)
    K, V, W, T = 10, 3, 4, 11
    S = rng.standard_normal((K, V))
    toks = _random_tokens(rng, "mamba2", K, V, T)
    Q = np.stack([t["q"] for t in toks])
    Km = np.stack([t["k"] for t in toks])
    Vm = np.stack([t["v"] for t in toks])
    a = np.array([t["a"] for t in toks])
    La = np.zeros((T, T))
    for t in range(T):
        for i in range(t + 1):
            La[t, i] = np.prod(a[i + 1:t + 1])
    Y = (La * (Q @ Km.T)) @ Vm + np.cumprod(a)[:, None] * (Q @ S)
    o = ItemOracle("mamba2", W, S)
    b = BatchOracle("mamba2", W, S[None], [None], [None])
    for t, tok in enumerate(toks):
        y, ye = o.read(tok["q"], tok["k"], tok["v"], tok["a"])
        yb, _ = b.read(tok["q"][None], tok["k"][None], tok["v"][None], np.array([tok["a"]]))
        np.testing.assert_allclose(ye, Y[t], rtol=0, atol=1e-12)
        np.testing.assert_allclose(y, Y[t], rtol=0, atol=1e-12)
        np.testing.assert_allclose(yb[0], Y[t], rtol=0, atol=1e-12)
        if o.j == W:
            o.flush()
            b.flush()


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_delta_rule_writes_value_at_key(kind):
    """With beta = 1 and a unit key, the delta rule stores v at k: S_t^T k_t = v_t,
    whatever the decay (for KDA this holds with the decay applied before the erase)."""
    rng = np.random.default_rng(5)
    K, V = 9, 4
    S = rng.standard_normal((K, V))
    o = ItemOracle(kind, 100, S)
    for tok in _random_tokens(rng, kind, K, V, 6, beta=1.0):
        o.read(tok["q"], tok["k"], tok["v"], tok["a"], 1.0)
        np.testing.assert_allclose(o.S.T @ tok["k"], tok["v"], rtol=0, atol=1e-12)


def test_kda_with_uniform_decay_is_gdn():
    rng = np.random.default_rng(6)
    K, V, W, r = 8, 3, 4, 2
    Om = rng.standard_normal((r, K))
    F = np.linalg.pinv(Om).T
    S = rng.standard_normal((K, V))
    a_ = ItemOracle("kda", W, S, Om, F)
    g_ = ItemOracle("gdn", W, S, Om, F)
    for tok in _random_tokens(rng, "kda", K, V, 10, a_uniform=True):
        ya, _ = a_.read(tok["q"], tok["k"], tok["v"], tok["a"], tok["beta"])
        yg, _ = g_.read(tok["q"], tok["k"], tok["v"], float(tok["a"][0]), tok["beta"])
        np.testing.assert_allclose(ya, yg, rtol=0, atol=1e-12)
        if a_.j == W:
            a_.flush()
            g_.flush()


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_beta_zero_only_decays(kind):
    """beta = 0: nothing is written or erased; y_t = S_init^T (prod of decays) q_t."""
    rng = np.random.default_rng(8)
    K, V, W = 7, 3, 3
    S = rng.standard_normal((K, V))
    o = ItemOracle(kind, W, S, rng.standard_normal((2, K)), rng.standard_normal((2, K)))
    d = np.ones(K)
    for tok in _random_tokens(rng, kind, K, V, 7, beta=0.0):
        _, ye = o.read(tok["q"], tok["k"], tok["v"], tok["a"], 0.0)
        d = d * (np.asarray(tok["a"]) if kind == "kda" else tok["a"])
        np.testing.assert_allclose(ye, S.T @ (d * tok["q"]), rtol=0, atol=1e-12)
        if o.j == W:
            o.flush()


@pytest.mark.parametrize("kind", KINDS)
def test_flushed_state_matches_wy_chunk_form(kind):
    """The state after a window equals the chunked (WY) form of the W updates:
    S_W = gamma_W * S_0 + sum_l ((gamma_W / gamma_l) * k_l) u_l^T with
    (I + L) U = diag(beta) (V - G), G_i = S_0^T (gamma_i * k_i),
    L_il = beta_i sum_c k_i[c] k_l[c] gamma_i[c] / gamma_l[c] (l < i),
    gamma_i the running product of decays."""
    rng = np.random.default_rng(9)
    K, V, W = 11, 4, 6
    S0 = rng.standard_normal((K, V))
    toks = _random_tokens(rng, kind, K, V, W)
    o = ItemOracle(kind, W, S0)
    for tok in toks:
        o.read(tok["q"], tok["k"], tok["v"], tok["a"], tok["beta"])
    Kw = np.stack([t["k"] for t in toks])
    Vw = np.stack([t["v"] for t in toks])
    beta = np.ones(W) if kind == "mamba2" else np.array([t["beta"] for t in toks])
    A = np.stack([np.broadcast_to(np.asarray(t["a"], float), (K,)) for t in toks])
    gam = np.cumprod(A, axis=0)  # gamma_1..gamma_W, per channel
    if kind == "mamba2":
        U = Vw
    else:
        G = (Kw * gam) @ S0
        L = np.zeros((W, W))
        for i in range(W):
            for l in range(i):
                L[i, l] = beta[i] * np.sum(Kw[i] * Kw[l] * gam[i] / gam[l])
        U = np.linalg.solve(np.eye(W) + L, beta[:, None] * (Vw - G))
    SW = gam[-1][:, None] * S0 + ((gam[-1] / gam) * Kw).T @ U
    np.testing.assert_allclose(o.S, SW, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# the two oracle modes agree
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c3", "c4"])
def test_item_and_batch_modes_agree(name):
    cfg = CONFIGS[name].with_batch(2)
    wl = Workload(cfg)
    hs = sorted(set([int(np.argmax(wl.ranks)), int(np.argmin(wl.ranks)), 0, cfg.H - 1]))
    items = [(b, h) for b in (0, 1) for h in hs]
    from oracle import gather_items, items_oracle
    bo = items_oracle(wl, items)
    its = []
    for (b, h) in items:
        r = int(wl.ranks[h])
        g = int(wl.groups[h])
        its.append(ItemOracle(cfg.kind, cfg.W, wl.state_item(b, h),
                              None if r == 0 else wl.basis[g, :r], None if r == 0 else wl.fmap(g, r)))
    for t in range(cfg.W + 3):
        st = gather_items(wl.step(t), items)
        yb, _ = bo.read(st["q"], st["k"], st["v"], st["a"], st["beta"])
        for i, it in enumerate(its):
            y, _ = it.read(st["q"][i], st["k"][i], st["v"][i], st["a"][i],
                           None if st["beta"] is None else st["beta"][i])
            np.testing.assert_allclose(yb[i], y, rtol=0, atol=1e-12 * max(1.0, np.abs(y).max()))
        if bo.j == cfg.W:
            bo.flush()
            for it in its:
                it.flush()


@pytest.mark.parametrize("kind", KINDS)
def test_intra_is_the_explicit_sum(kind):
    """intra_j = sum_{i<=j} beta_i v_i (k_i^T M_{i+1}^T ... M_j^T q_j)."""
    rng = np.random.default_rng(10)
    K, V, W = 6, 3, 5
    S = rng.standard_normal((K, V))
    Om = rng.standard_normal((2, K))
    F = np.linalg.pinv(Om).T
    o = ItemOracle(kind, W, S, Om, F)
    toks = _random_tokens(rng, kind, K, V, W)
    for j, tok in enumerate(toks, start=1):
        y, ye = o.read(tok["q"], tok["k"], tok["v"], tok["a"], tok["beta"])
        qt = o.P.T @ tok["q"]
        intra_oracle = y - o.Z.T @ (o.fmap @ qt)
        want = np.zeros(V)
        for i in range(1, j + 1):
            u = tok["q"].copy()
            for m in range(j, i, -1):
                u = transition(kind, toks[m - 1]["a"], toks[m - 1]["beta"], toks[m - 1]["k"]).T @ u
            bi = 1.0 if kind == "mamba2" else toks[i - 1]["beta"]
            want += bi * toks[i - 1]["v"] * (toks[i - 1]["k"] @ u)
        np.testing.assert_allclose(intra_oracle, want, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# state-access traffic
# ---------------------------------------------------------------------------
def _traffic_oracle(ranks, K=128, V=80, W=16, seed=9):
    """A BatchOracle over items of the given ranks (0 = dense), random orthonormal
    basis rows, run through one full window and its flush."""
    rng = np.random.default_rng(seed)
    Om, _ = np.linalg.qr(rng.standard_normal((K, K)))
    Om = Om.T
    n = len(ranks)
    omega = [None if r == 0 else Om[:r] for r in ranks]
    fmap = [None if r == 0 else Om[:r] for r in ranks]
    orc = BatchOracle("mamba2", W, 0.02 * rng.standard_normal((n, K, V)), omega, fmap)
    start = dict(orc.traffic)
    per_read = []
    for _ in range(W):
        before = dict(orc.traffic)
        k = rng.standard_normal((n, K))
        orc.read(rng.standard_normal((n, K)), k / np.linalg.norm(k, axis=1, keepdims=True),
                 rng.standard_normal((n, V)), rng.uniform(0.9, 1.0, n))
        per_read.append({key: orc.traffic[key] - before[key] for key in before})
    orc.flush()
    return orc, start, per_read


def test_sketch_read_traffic_is_rank_over_K():
    """A decode read of a rank-r head moves r/K of the state bytes that a dense
    (full-state) read moves: Z is r x V, S is K x V."""
    K, V = 128, 80
    _, _, de = _traffic_oracle([0], K=K, V=V)
    for r in (1, 6, 8, 16, 49):
        _, _, sk = _traffic_oracle([r], K=K, V=V)
        for a, b in zip(sk, de):
            assert a["S_read"] == 0 and a["S_write"] == 0 and a["Z_write"] == 0
            assert b["Z_read"] == 0 and b["S_write"] == 0
            assert Fraction(a["Z_read"], b["S_read"]) == Fraction(r, K)
    # heads of mixed ranks in one launch: each moves its own r/K, not the largest
    ranks = [1, 6, 8, 16, 49, 0, 0]
    _, _, mixed = _traffic_oracle(ranks, K=K, V=V)
    for a in mixed:
        assert Fraction(a["Z_read"], de[0]["S_read"]) == Fraction(sum(ranks), K)
        assert a["S_read"] == 2 * de[0]["S_read"]


def test_state_traffic_about_ten_times_lower_at_mean_rank_8():
    """The Abstract of "SketchSSM: Write to the Full State, Read from a Compact
    Sketch" reports about 10x less state-access traffic at a mean sketch rank
    of 8.  Against the standard decode, which reads and writes the whole state
    for every token, one window of W = 16 tokens of rank-8 heads (Nano shape,
    K = 128) moves 2KW / (rW + 2K + r) = 10.45x fewer state bytes."""
    K, V, W, r, n = 128, 80, 16, 8, 4
    orc, start, _ = _traffic_oracle([r] * n, K=K, V=V, W=W)
    moved = sum(orc.traffic[key] - start[key] for key in orc.traffic)
    standard = W * n * 2 * K * V * 4
    ratio = standard / moved
    assert ratio == pytest.approx(2 * K * W / (r * W + 2 * K + r), rel=1e-12)
    assert 9.5 < ratio < 11.5
    # dense heads gain nothing: their reads are full state reads
    orc, start, _ = _traffic_oracle([0] * n, K=K, V=V, W=W)
    moved = sum(orc.traffic[key] - start[key] for key in orc.traffic)
    assert standard / moved == pytest.approx(2 * W / (W + 2), rel=1e-12)
