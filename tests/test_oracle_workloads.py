"""Pins of the oracle's workload-level steps: SelectInfer base/dynamic/union
selection, the SpAx three-tier product and its 4-bit codec, the ReLU-sparse
MoE expert, and batched decode over a union."""
import json
import os

import numpy as np
import pytest

import oracle
from activation_sparse_decode_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16(values):
    return synth.f32_to_bf16_bits(np.asarray(values, dtype=np.float32))


# ------------------------------------------------------------------ SelectInfer (hand-derived fixture)

def test_selectinfer_tiny_fixture():
    with open(os.path.join(GOLDEN, "selectinfer_tiny.json")) as fh:
        g = json.load(fh)
    calib = np.array(g["calib_acts"], dtype=np.float32)
    s, base = oracle.base_set(calib, g["delta"])
    assert s.tolist() == g["expected_scores"]
    assert base.tolist() == g["expected_base"]
    prompt = np.array(g["prompt_acts"], dtype=np.float32)
    for t, exp in enumerate(g["expected_token_sets"]):
        assert oracle.rank_range(oracle.key_abs(prompt[t]), 0, g["alpha"]).tolist() == exp
    counts, dyn = oracle.dynamic_set(prompt, g["alpha"], g["beta"])
    assert counts.tolist() == g["expected_counts"]
    assert dyn.tolist() == g["expected_dynamic"]
    assert oracle.union(base, dyn).tolist() == g["expected_union"]


def test_selectinfer_invariants():
    rng = np.random.default_rng(21)
    N, T = 500, 40
    alpha, beta, delta = oracle.count_of(30, N), oracle.count_of(20, N), oracle.count_of(20, N)
    calib = rng.standard_normal((64, N)).astype(np.float32)
    prompt = rng.standard_normal((T, N)).astype(np.float32)
    _, base = oracle.base_set(calib, delta)
    counts, dyn = oracle.dynamic_set(prompt, alpha, beta)
    assert counts.sum() == T * alpha
    U = oracle.union(base, dyn)
    assert max(base.size, dyn.size) <= U.size <= base.size + dyn.size
    assert set(base.tolist()) | set(dyn.tolist()) == set(U.tolist())
    # an empty base set leaves the prompt-only (CoreInfer-style) dynamic set
    assert oracle.union(np.zeros(0, np.int32), dyn).tolist() == dyn.tolist()


def test_decode_over_full_set_is_dense():
    rng = np.random.default_rng(22)
    N, d = 48, 32
    Wg, Wu, WdT = (synth.weight_bf16(0, 9, 3, 0, t, N, d) for t in range(3))
    h = rng.standard_normal(d).astype(np.float32)
    a_full, y_full = oracle.decode_over_set(Wg, Wu, WdT, h, np.arange(N))
    A_dense, Y_dense = oracle.dense_ffn(Wg, Wu, WdT, h[None, :])
    assert np.array_equal(a_full, A_dense[0])
    np.testing.assert_allclose(y_full, Y_dense[0], rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------------ SpAx codec and tiers

def test_encoder_exact_on_grid():
    # columns built on a 4-bit grid with fp16-exact zero/scale decode exactly
    rng = np.random.default_rng(23)
    n_in, n_out = 6, 32
    seg = [0, 16, 24, 32]
    zero_s = [-1.0, -0.5, -0.25]
    step_s = [0.125, 0.0625, 0.03125]
    W = np.zeros((n_in, n_out), dtype=np.float32)
    for s in range(3):
        lo, hi = seg[s], seg[s + 1]
        q = rng.integers(0, 16, size=(n_in, hi - lo))
        q[:, 0], q[:, 1] = 0, 15
        W[:, lo:hi] = zero_s[s] + step_s[s] * q
    Wb = bf16(W)
    scale, zero, q = oracle.encode_4bit(Wb, seg)
    for s in range(3):
        assert np.all(zero[:, s] == np.float16(zero_s[s]))
        assert np.all(scale[:, s] == np.float16(step_s[s]))
    assert np.array_equal(oracle.decode_4bit(scale, zero, q, seg), W.astype(np.float64))


def test_encoder_error_bound_and_ranges():
    rng = np.random.default_rng(24)
    n_in, n_out = 40, 96
    seg = [0, 64, 80, 96]
    Wb = synth.weight_bf16(0, 9, 4, 0, 6, n_in, n_out)
    Wb[3, 64:80] = bf16(np.full(16, 0.01))           # constant segment -> scale 0
    scale, zero, q = oracle.encode_4bit(Wb, seg)
    assert q.max() <= 15
    assert np.all(q[3, 64:80] == 0) and scale[3, 1] == 0
    W = oracle.widen_bf16(Wb)
    W_hat = oracle.decode_4bit(scale, zero, q, seg)
    for s in range(3):
        lo, hi = seg[s], seg[s + 1]
        w = W[:, lo:hi]
        sc = scale[:, s].astype(np.float64)
        rng_exact = w.max(axis=1) - w.min(axis=1)
        slack = (np.abs(zero[:, s].astype(np.float64) - w.min(axis=1))
                 + 15 * np.abs(sc - rng_exact / 15) + 1e-12)
        err = np.abs(w - W_hat[:, lo:hi]).max(axis=1)
        assert np.all(err <= 0.5 * sc + slack)
        # the segment minimum codes to 0 and the maximum to 15 (or 14/15 after fp16 rounding)
        qmin = q[:, lo:hi].min(axis=1)
        qmax = q[:, lo:hi].max(axis=1)
        live = sc > 0
        assert np.all(qmin[live] == 0) and np.all(qmax[live] >= 14)


def test_tier_sets_partition_and_order():
    rng = np.random.default_rng(25)
    x = (rng.standard_normal(200) * np.exp(rng.standard_normal(200))).astype(np.float32)
    top, mid = oracle.tier_sets(x, 30, 70)
    assert top.size == 30 and mid.size == 70 and np.intersect1d(top, mid).size == 0
    assert np.abs(x[top]).min() >= np.abs(x[mid]).max()
    skipped = np.setdiff1d(np.arange(200), np.concatenate([top, mid]))
    assert np.abs(x[mid]).min() >= np.abs(x[skipped]).max()


# ------------------------------------------------------------------ SelectInfer selective loading
def test_selective_loading_fixture():
    g = json.load(open(os.path.join(GOLDEN, "selectinfer_loading_tiny.json")))
    s_task = np.array(g["s_task"], np.float32)
    s_model = np.array(g["s_model"], np.float32)
    base, loaded = oracle.selective_loading(s_task, s_model, g["delta"], g["gamma"])
    assert base.tolist() == g["expected_base"]
    assert loaded.tolist() == g["expected_loaded"]
    pos = oracle.loaded_positions(loaded, base)
    assert pos.tolist() == g["expected_static_positions"]
    counts = np.array(g["counts_over_loaded"])
    for phi, exp in g["phi_cases"]:
        assert oracle.fill_to_phi(pos, counts, phi).tolist() == exp, phi
    assert loaded[oracle.fill_to_phi(pos, counts, 3)].tolist() == g["expected_ids_phi3"]
    r = oracle.modified_layers(g["layers"], g["first"], g["last"])
    assert [r[0], r[-1]] == g["expected_modified"] and len(r) == 21


def test_modified_layers_range_forms():
    # last <= 0 counts from the end, last > 0 is an exclusive bound
    assert list(oracle.modified_layers(28, 0, 0)) == list(range(28))
    assert list(oracle.modified_layers(28, 5, -2)) == list(range(5, 26))
    assert list(oracle.modified_layers(6, 1, -1)) == [1, 2, 3, 4]
    assert list(oracle.modified_layers(28, 4, 27)) == list(range(4, 27))
    assert list(oracle.modified_layers(3, 3, 0)) == []


def brute_fill(start, values, total):
    """Walk the entries by (|value| desc, index asc) with Python floats,
    adding those not yet present, until ``total`` are present."""
    chosen = sorted(set(start))
    order = sorted(range(len(values)), key=lambda n: (-abs(float(values[n])), n))
    for n in order:
        if len(chosen) >= total:
            break
        if n not in chosen:
            chosen = sorted(chosen + [n])
    return chosen


def test_selective_loading_brute_force():
    rng = np.random.default_rng(29)
    for trial in range(300):
        N = int(rng.integers(1, 11))
        s_task = rng.integers(0, 4, N).astype(np.float32) * np.float32(0.5)
        s_model = rng.integers(0, 4, N).astype(np.float32)        # ties and zeros
        delta = int(rng.integers(0, N + 1))
        gamma = int(rng.integers(delta, N + 2))
        base, loaded = oracle.selective_loading(s_task, s_model, delta, gamma)
        exp_base = sorted(range(N), key=lambda n: (-float(s_task[n]), n))[:delta]
        assert base.tolist() == sorted(exp_base), trial
        assert loaded.tolist() == brute_fill(exp_base, s_model, gamma), trial
        assert loaded.size == min(gamma, N) and np.isin(base, loaded).all()
        counts = rng.integers(0, 3, loaded.size)
        static = oracle.loaded_positions(loaded, base)
        phi = int(rng.integers(0, loaded.size + 2))
        U = oracle.fill_to_phi(static, counts, phi)
        assert U.tolist() == brute_fill(static.tolist(), counts, phi), trial
        assert U.size == max(static.size, min(phi, loaded.size))


def test_selective_loading_special_cases():
    rng = np.random.default_rng(30)
    N = 500
    s = (rng.random(N) * 10).astype(np.float32)
    s2 = (rng.random(N) * 10).astype(np.float32)
    # the same scores for both: the loaded set is the top gamma of that ranking
    base, loaded = oracle.selective_loading(s, s, 150, 350)
    assert np.array_equal(loaded, oracle.rank_range(oracle.key_abs(s), 0, 350))
    # gamma = delta: only the base is loaded; gamma = N: everything
    base, loaded = oracle.selective_loading(s, s2, 150, 150)
    assert np.array_equal(loaded, base)
    assert np.array_equal(oracle.selective_loading(s, s2, 150, N)[1], np.arange(N))
    # base and secondary are disjoint and together fill gamma
    base, loaded = oracle.selective_loading(s, s2, 150, 350)
    sec = np.setdiff1d(loaded, base)
    assert sec.size == 200
    rest = np.setdiff1d(np.arange(N), loaded)
    assert s2[sec].min() >= s2[rest].max()
    # fill to phi: counts ranked like the static set give the plain top phi
    static = oracle.rank_range(oracle.key_abs(s), 0, 100)
    cnt = (s * 100).astype(np.int64)
    assert np.array_equal(oracle.fill_to_phi(static, cnt, 180),
                          oracle.rank_range(cnt.astype(np.uint32), 0, 180))
    # phi below the static size leaves the static set; union of static and top-beta
    # frequency set when no static neuron is among the frequent ones
    assert np.array_equal(oracle.fill_to_phi(static, cnt, 50), static)
    cnt2 = cnt.copy()
    cnt2[static] = 0
    U = oracle.fill_to_phi(static, cnt2, 180)
    assert np.array_equal(U, oracle.union(static, oracle.rank_range(cnt2.astype(np.uint32), 0, 80)))


# ------------------------------------------------------------------ PowerInfer-2 online predictor
def test_predictor_logits_integer_bruteforce():
    rng = np.random.default_rng(31)
    W = rng.integers(-4, 5, (7, 16)).astype(np.float32)
    h = rng.integers(-3, 4, 16).astype(np.float64)
    b = rng.integers(-5, 6, 7).astype(np.float64)
    got = oracle.predictor_logits(bf16(W), b, h)
    for k in range(7):
        assert got[k] == sum(int(W[k, i]) * int(h[i]) for i in range(16)) + int(b[k])
    assert np.array_equal(oracle.predictor_logits(bf16(W), None, h), got - b)


def exact_above(z: float, theta: float) -> bool:
    """sigma(z) > theta at 60 significant digits."""
    import decimal
    with decimal.localcontext() as ctx:
        ctx.prec = 60
        zd, td = decimal.Decimal(float(z)), decimal.Decimal(float(theta))
        return 1 / (1 + (-zd).exp()) > td


def test_predicted_clusters_exact_decision():
    rng = np.random.default_rng(32)
    for theta in (float(np.float32(0.45)), 0.5, float(np.float32(0.3)), float(np.float32(0.9))):
        t = np.log(theta / (1 - theta))
        near = np.float32(t)
        z = [near]
        for _ in range(4):                       # fp32 neighbours on both sides of the logit
            z = [np.nextafter(z[0], np.float32(-10), dtype=np.float32)] + z + \
                [np.nextafter(z[-1], np.float32(10), dtype=np.float32)]
        z = np.concatenate([np.array(z, np.float32),
                            rng.uniform(-4, 4, 200).astype(np.float32), np.float32([0.0])])
        got = oracle.predicted_clusters(z.astype(np.float64), theta)
        exp = [k for k in range(z.size) if exact_above(z[k], theta)]
        assert got.tolist() == exp, theta
    # sigma(0) = 1/2: strictly above theta = 1/2 needs z > 0
    z = np.array([0.0, 1e-30, -1e-30], np.float64)
    assert oracle.predicted_clusters(z, 0.5).tolist() == [1]
    # the sets shrink as theta grows
    z = rng.standard_normal(500)
    prev = None
    for theta in (0.1, 0.3, 0.45, 0.5, 0.7, 0.95):
        cur = set(oracle.predicted_clusters(z, theta).tolist())
        assert prev is None or cur <= prev
        prev = cur


def test_predicted_expert_special_cases():
    rng = np.random.default_rng(33)
    N, d, S = 256, 64, 32
    Wg = synth.weight_bf16(0, 9, 1, 0, 0, N, d)
    Wu = synth.weight_bf16(0, 9, 1, 0, 1, N, d)
    WdT = synth.weight_bf16(0, 9, 1, 0, 2, N, d)
    h = rng.standard_normal(d)
    tau = oracle.relu_threshold(h, 1.2815515655446004, 0.02)
    ref = oracle.relu_expert(Wg, Wu, WdT, h, tau, S)
    # all clusters, or exactly the active ones: the ReLU expert's output
    for cl in (np.arange(N // S), ref["clusters"]):
        got = oracle.predicted_expert(Wg, Wu, WdT, h, tau, cl, S)
        np.testing.assert_allclose(got["y"], ref["y"], rtol=1e-6, atol=1e-9)
    # an inactive cluster contributes exactly nothing; a missed active one its own rows
    inactive = np.setdiff1d(np.arange(N // S), ref["clusters"])
    if inactive.size and ref["clusters"].size:
        more = oracle.predicted_expert(Wg, Wu, WdT, h, tau, np.union1d(ref["clusters"], inactive[:1]), S)
        act = oracle.predicted_expert(Wg, Wu, WdT, h, tau, ref["clusters"], S)
        assert np.array_equal(more["y"], act["y"]) or np.allclose(more["y"], act["y"], rtol=1e-15)
        assert not np.any(more["a32"][np.isin(more["rows"], oracle.expand_clusters(inactive[:1], S))])
    # no cluster predicted: nothing computed
    none = oracle.predicted_expert(Wg, Wu, WdT, h, tau, np.zeros(0, np.int32), S)
    assert none["rows"].size == 0 and not np.any(none["y"])


def test_relu_glu_rows_worked_example():
    # gate rows (1, 2) and (-1, 0.5), up rows (3, 0) and (0, 4), h = (1, 1),
    # tau = 1: gate dots 3 and -0.5, up dots 3 and 4, so a = (max(3 - 1, 0) * 3,
    # max(-0.5 - 1, 0) * 4) = (6, 0).  A dropped threshold gives 9 for row 0,
    # swapped gate and up rows -1.5 for row 1, a wrong row subset the other value.
    Wg = bf16([[1.0, 2.0], [-1.0, 0.5]])
    Wu = bf16([[3.0, 0.0], [0.0, 4.0]])
    h = np.array([1.0, 1.0])
    assert oracle.relu_glu_rows(Wg, Wu, h, 1.0, np.array([0, 1])).tolist() == [6.0, 0.0]
    assert oracle.relu_glu_rows(Wg, Wu, h, 1.0, np.array([1, 0])).tolist() == [0.0, 6.0]
    assert oracle.relu_glu_rows(Wg, Wu, h, 1.0, np.array([1])).tolist() == [0.0]
    # tau = -1 lets row 1's gate through: max(-0.5 + 1, 0) * 4 = 2
    assert oracle.relu_glu_rows(Wg, Wu, h, -1.0, np.array([0, 1])).tolist() == [12.0, 2.0]


def test_active_clusters_bruteforce():
    rng = np.random.default_rng(41)
    for trial in range(100):
        c = int(rng.choice([1, 2, 4, 32]))
        n = c * int(rng.integers(1, 40))
        r = np.maximum(rng.standard_normal(n), 0.0).astype(np.float32)
        if trial % 3 == 0:   # whole clusters at zero, some with a single nonzero value
            dead = rng.random(n // c) < 0.6
            r.reshape(-1, c)[dead] = 0.0
            lone = np.flatnonzero(dead)[: max(1, dead.sum() // 3)]
            r.reshape(-1, c)[lone, rng.integers(0, c)] = np.float32(1e-30)
        if trial == 7:
            r[:] = 0.0
        expected = [q for q in range(n // c) if any(v != 0.0 for v in r[q * c:(q + 1) * c])]
        assert oracle.active_clusters(r, c).tolist() == expected, (trial, c, n)


# ------------------------------------------------------------------ WiSparse weight-aware saliency
def test_row_norms_closed_forms():
    d = 16
    const = np.full((3, d), 0.0, np.float32)
    const[0], const[1], const[2] = 0.5, -3.0, 0.0
    assert oracle.row_norms(bf16(const)).tolist() == [0.5 * 4, 3.0 * 4, 0.0]
    # Pythagorean rows, placed in different columns and in a non-square W^T
    W = np.zeros((4, 7), np.float32)
    W[0, [0, 6]] = [3, 4]
    W[1, [1, 2, 5]] = [-2, 3, 6]
    W[2, 3] = -9
    W[3, :] = np.arange(1, 8)
    got = oracle.row_norms(bf16(W))
    np.testing.assert_array_equal(got[:3], [5.0, 7.0, 9.0])
    assert got[3] == pytest.approx(np.sqrt(sum(i * i for i in range(1, 8))), rel=1e-15)
    # one norm per input channel (row of W^T), not per output
    assert oracle.row_norms(bf16(np.ones((5, 9), np.float32))).shape == (5,)


def test_weighted_key_fp32_product_brute_force():
    rng = np.random.default_rng(27)
    for trial in range(200):
        n = int(rng.integers(1, 12))
        x = rng.integers(-20, 21, n).astype(np.float32)
        w = rng.integers(0, 16, n).astype(np.float32)
        keys = oracle.weighted_key(x, w)
        sal = [abs(int(a)) * int(b) for a, b in zip(x, w)]        # exact in fp32
        order = sorted(range(n), key=lambda j: (-sal[j], j))
        k_top = int(rng.integers(0, n + 1))
        k_mid = int(rng.integers(0, n + 1 - k_top))
        top, mid = oracle.weighted_tier_sets(x, w, k_top, k_mid)
        assert top.tolist() == sorted(order[:k_top]), (trial, x, w)
        assert mid.tolist() == sorted(order[k_top:k_top + k_mid]), (trial, x, w)
        assert all(int(keys[j]) == np.float32(sal[j]).view(np.uint32) for j in range(n))


def test_weighted_key_special_cases():
    rng = np.random.default_rng(28)
    x = (rng.standard_normal(300) * np.exp(rng.standard_normal(300))).astype(np.float32)
    # unit norms, and a power-of-two norm for every channel: the |x| tiers
    for c in (1.0, 0.25, 8.0):
        for got, ref in zip(oracle.weighted_tier_sets(x, np.full(300, c, np.float32), 40, 90),
                            oracle.tier_sets(x, 40, 90)):
            assert np.array_equal(got, ref)
    # the sign of x does not matter
    for got, ref in zip(oracle.weighted_tier_sets(-x, np.ones(300, np.float32), 40, 90),
                        oracle.tier_sets(x, 40, 90)):
        assert np.array_equal(got, ref)
    # a zero-norm channel ranks with the zero activations, after every live one
    w = np.ones(300, np.float32)
    big = int(np.argmax(np.abs(x)))
    w[big] = 0.0
    top, _ = oracle.weighted_tier_sets(x, w, 299, 0)
    assert big not in top.tolist() and top.size == 299
    # the norm reorders: |x| prefers channel 1, |x| * norm channel 0
    top, mid = oracle.weighted_tier_sets(np.array([1.0, 2.0], np.float32),
                                         np.array([3.0, 1.0], np.float32), 1, 1)
    assert top.tolist() == [0] and mid.tolist() == [1]
    assert oracle.tier_sets(np.array([1.0, 2.0], np.float32), 1, 1)[0].tolist() == [1]


def test_weighted_key_is_rounded_to_fp32():
    # channel 0: (1 + 2^-22) * 1 exactly; channel 1: (1 + 2^-23)^2 = 1 + 2^-22 + 2^-46,
    # larger in exact arithmetic but the same fp32 value, so the tie goes to index 0
    e23, e22 = np.float32(2.0 ** -23), np.float32(2.0 ** -22)
    x = np.array([1 + e22, 1 + e23], np.float32)
    w = np.array([1.0, 1 + e23], np.float32)
    assert (1 + 2.0 ** -23) ** 2 > 1 + 2.0 ** -22
    keys = oracle.weighted_key(x, w)
    assert keys[0] == keys[1]
    assert oracle.weighted_tier_sets(x, w, 1, 0)[0].tolist() == [0]


def test_tiered_special_cases():
    rng = np.random.default_rng(26)
    n_in, n_out = 64, 48
    seg = [0, 32, 40, 48]
    WT = synth.weight_bf16(0, 9, 5, 0, 6, n_in, n_out)
    x = rng.standard_normal(n_in).astype(np.float32)
    scale, zero, q = oracle.encode_4bit(WT, seg)
    dense = oracle.widen_bf16(WT).T @ x.astype(np.float64)
    # all columns in the top tier: the dense product
    y = oracle.tiered_gemv(WT, scale, zero, q, seg, x, np.arange(n_in), np.zeros(0, np.int32))
    np.testing.assert_allclose(y, dense, rtol=1e-12, atol=1e-15)
    # k_mid = 0: the plain gathered product over the top columns
    top, mid = oracle.tier_sets(x, 10, 0)
    y = oracle.tiered_gemv(WT, scale, zero, q, seg, x, top, mid)
    np.testing.assert_allclose(y, oracle.down_gather(WT, top, x[top]), rtol=1e-12, atol=1e-15)
    # all columns in the middle tier: the dense product with reconstructed columns
    y = oracle.tiered_gemv(WT, scale, zero, q, seg, x, np.zeros(0, np.int32), np.arange(n_in))
    W_hat = oracle.decode_4bit(scale, zero, q, seg)
    manual = np.zeros(n_out)
    for j in range(n_in):
        manual += W_hat[j] * float(x[j])
    np.testing.assert_allclose(y, manual, rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------------ ReLU-sparse MoE

def test_route_top2_bruteforce():
    rng = np.random.default_rng(27)
    for trial in range(200):
        logits = rng.standard_normal(8).astype(np.float32)
        if trial % 4 == 0:
            logits[rng.integers(0, 8)] = logits[rng.integers(0, 8)]   # ties
        experts, w = oracle.route_top2(logits)
        order = sorted(range(8), key=lambda e: (-float(logits[e]), e))
        assert experts.tolist() == sorted(order[:2])
        v = [float(logits[e]) for e in experts]
        z = [np.exp(t - max(v)) for t in v]
        assert w.tolist() == pytest.approx([t / sum(z) for t in z], rel=1e-14)
        assert w.sum() == pytest.approx(1.0, rel=1e-15)


def test_relu_expert_sparse_equals_dense():
    rng = np.random.default_rng(28)
    N, d, S = 256, 64, 32
    Wg = synth.clustered_gate_bf16(0, 9, 0, 0, N, d, S)
    Wu = synth.weight_bf16(0, 9, 0, 0, synth.T_UP, N, d)
    WdT = synth.weight_bf16(0, 9, 0, 0, synth.T_DOWN, N, d)
    h = rng.standard_normal(d).astype(np.float32)
    tau = oracle.relu_threshold(h, 1.2815515655446004, 0.02)
    res = oracle.relu_expert(Wg, Wu, WdT, h, tau, S)
    # dense ReGLU over all neurons
    r = np.maximum(oracle.row_dots(Wg, h) - tau, 0.0).astype(np.float32)
    a = (r.astype(np.float64) * oracle.row_dots(Wu, h)).astype(np.float32)
    y_dense = oracle.widen_bf16(WdT).T @ a.astype(np.float64)
    np.testing.assert_allclose(res["y"], y_dense, rtol=1e-12, atol=1e-15)
    skipped = np.setdiff1d(np.arange(N), res["rows"])
    assert np.all(r[skipped] == 0)
    for c in range(N // S):
        active = bool(np.any(r[c * S:(c + 1) * S] > 0))
        assert active == (c in res["clusters"].tolist())


def test_relu_threshold_sparsity():
    rng = np.random.default_rng(29)
    N, d = 4096, 512
    Wg = synth.weight_bf16(0, 9, 1, 0, 0, N, d)
    h = rng.standard_normal(d).astype(np.float32)
    tau = oracle.relu_threshold(h, 1.2815515655446004, 0.02)
    frac = np.mean(oracle.relu_gate(Wg, h, tau) > 0)
    assert 0.08 < frac < 0.12           # ~10% nonzero (1 - Phi(1.2816) = 0.1)


# ------------------------------------------------------------------ batched decode

def test_batched_union_reduces_to_single_token():
    rng = np.random.default_rng(30)
    N, d, B, keep = 80, 40, 4, 32
    Wg, Wu, WdT = (synth.weight_bf16(0, 9, 6, 0, t, N, d) for t in range(3))
    X = rng.standard_normal((B, d)).astype(np.float32)
    res = oracle.batched_union_decode(Wg, Wu, WdT, X, keep)
    sets = []
    for b in range(B):
        single = oracle.sparse_swiglu_layer(Wg, Wu, WdT, X[b], keep)
        assert np.array_equal(single["idx"], res["S"][b])
        np.testing.assert_allclose(res["Y"][b], single["y"], rtol=1e-13, atol=1e-15)
        sets.append(set(single["idx"].tolist()))
    assert set(res["U"].tolist()) == set().union(*sets)
    # a neuron of U outside S_b must not feed token b: masking it by hand
    b = 0
    a_masked = np.where(np.isin(np.arange(N), res["S"][b]), res["A32"][b], 0.0)
    y_union = oracle.down_gather(WdT, res["U"], a_masked[res["U"]])
    np.testing.assert_allclose(y_union, res["Y"][b], rtol=1e-12, atol=1e-15)
