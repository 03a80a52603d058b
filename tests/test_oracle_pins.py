"""Pins of the CPU oracle to what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a worked
example printed on the pages (fixtures under tests/golden/, each citing its
page and section), a closed form, an invariant, a special case that reduces
to a library routine, or an independent brute-force evaluation.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synthetic
from conftest import read_golden


def f32cfg(**kw):
    cfg = dict(d=4, L=0, n=4, k=2, F=4, kind="relu2", act="f32", weights="f32", router_w="f32",
               in_norm="none", expert_norm="none", res_gate="none", eps_in=0.0, eps_expert=0.0,
               bias_in_weights=0)
    cfg.update(kw)
    return cfg


# ---------------------------------------------------------------------------
# Norms: worked example of C_gamma vs I_gamma (normalization-orders section)
# ---------------------------------------------------------------------------

def test_rmsnorm_orders_worked_example():
    g = read_golden("rmsnorm_orders.txt")
    x, gamma = np.array(g["x"]), np.array(g["gamma"], np.float32)
    C = oracle.rms_centered(x, gamma, 0.0)
    np.testing.assert_allclose(C, g["C"], rtol=0, atol=1e-15)
    I_ = oracle.rms_input_scaled(x, gamma, 0.0)
    expect = np.array(g["I_num"]) / math.sqrt(g["I_den_sq"][0])
    np.testing.assert_allclose(I_, expect, rtol=0, atol=1e-15)
    # rounding the scaled vector (2,1) to bf16 is exact, so the bf16 form agrees
    np.testing.assert_allclose(oracle.rms_input_scaled(x, gamma, 0.0, act="bf16"), expect, atol=1e-15)
    # collinear but not equal
    assert abs(C[0] / C[1] - I_[0] / I_[1]) < 1e-12 and not np.allclose(C, I_)


def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(37)
    # gamma = 0 and eps = 0: both orders reduce to x / rms(x), with mean square 1 afterwards
    for f in (lambda v: oracle.rms_centered(v, None, 0.0), lambda v: oracle.rms_input_scaled(v, None, 0.0)):
        r = f(x)
        assert abs(np.mean(r * r) - 1.0) < 1e-14
        np.testing.assert_allclose(r, x / np.sqrt(np.mean(x * x)), rtol=1e-14)
    # epsilon enters under the root: a constant vector c gives c / sqrt(c^2 + eps)
    c = np.full(8, 0.3)
    np.testing.assert_allclose(oracle.rms_centered(c, None, 0.5), c / math.sqrt(0.09 + 0.5), rtol=1e-15)
    # C scales after normalising: output of a gain g is (1+g) times the gain-free output
    gam = rng.standard_normal(37).astype(np.float32) * 0.1
    np.testing.assert_allclose(oracle.rms_centered(x, gam, 1e-3),
                               (1 + gam.astype(np.float64)) * oracle.rms_centered(x, None, 1e-3), rtol=1e-14)


def test_input_scaled_rounds_scaled_vector_to_input_dtype():
    # The scaled vector is rounded to bf16 before the reduction: pick values where that matters.
    x = np.array([1.0 + 2 ** -8, 1.0, 3.0, -2.0])   # 1+2^-8 is a bf16 tie: rounds to 1.0 (even)
    gamma = np.zeros(4, np.float32)
    r = oracle.rms_input_scaled(x, gamma, 0.0, act="bf16")
    s = np.array([1.0, 1.0, 3.0, -2.0])
    np.testing.assert_allclose(r, s / np.sqrt(np.mean(s * s)), rtol=1e-15)


# ---------------------------------------------------------------------------
# bf16 rounding used by the oracle vs torch's conversion (a library routine)
# ---------------------------------------------------------------------------

def test_round_bf16_matches_library_and_ties():
    rng = np.random.default_rng(1)
    vals = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000),
                           [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 2 ** -130, 3.0e-39]])
    ours = np.array([oracle.round_bf16(v) for v in vals])
    ref = torch.tensor(vals.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    # torch rounds via float32 first; for these values that first step is exact or harmless
    np.testing.assert_array_equal(ours, ref)
    assert oracle.round_bf16(1.0 + 2 ** -8) == 1.0            # tie to even (down)
    assert oracle.round_bf16(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6  # tie to even (up)


# ---------------------------------------------------------------------------
# Gate: worked example, invariants and special cases ("The gate")
# ---------------------------------------------------------------------------

def _router_layer(H):
    """A layer whose router logits equal H for the input x = e_0."""
    n = len(H)
    x = np.zeros((1, n), np.float32)
    x[0, 0] = 1.0
    W = np.zeros((n, n), np.float32)
    W[:, 0] = H
    return x, W


def test_topk_softmax_worked_example():
    g = read_golden("topk_softmax.txt")
    H, k = np.array(g["H"]), int(g["k"][0])
    G = oracle.gate_dense(H, k)
    np.testing.assert_allclose(G, g["G_printed"], atol=5e-4)          # the page's three places
    np.testing.assert_allclose(G[:2], [1 / (1 + math.exp(-1)), 1 / (1 + math.exp(1))], rtol=1e-15)
    assert G[2] == 0.0 and G[3] == 0.0
    # the same numbers through the full forward: a router whose logits are H
    x, W = _router_layer(H)
    n = len(H)
    cfg = f32cfg(d=n, n=n, k=k, F=2)
    t = {"x": x, "router_w": W, "w1": np.zeros((n, 2, n), np.float32), "w2": np.zeros((n, n, 2), np.float32)}
    r = oracle.forward(cfg, t)
    assert list(r["idx"][0]) == [0, 1]
    np.testing.assert_allclose(r["w"][0], G[:2], rtol=1e-15)


@pytest.mark.parametrize("n,k", [(8, 2), (256, 8), (5, 5), (7, 1)])
def test_gate_invariants(n, k):
    rng = np.random.default_rng(n * 100 + k)
    for _ in range(20):
        H = rng.standard_normal(n) * 3
        G = oracle.gate_dense(H, k)
        assert (G >= 0).all()
        assert abs(G.sum() - 1.0) < k * 2.0 ** -52 * 4
        assert (G > 0).sum() == k
        # the kept entries are exactly the k largest
        kept = set(np.flatnonzero(G))
        assert kept == set(np.argsort(-H, kind="stable")[:k])


def test_gate_special_cases():
    rng = np.random.default_rng(3)
    H = rng.standard_normal(9)
    # k = 1: the single survivor gets weight exactly 1
    G = oracle.gate_dense(H, 1)
    assert G.max() == 1.0 and G.argmax() == np.argmax(H)
    # k = n: the ordinary softmax
    np.testing.assert_allclose(oracle.gate_dense(H, 9), scipy.special.softmax(H), rtol=1e-14)
    # exact ties: lower expert id first, equal weights 1/k
    idx, margin = oracle.topk(np.zeros(16), 4)
    assert list(idx) == [0, 1, 2, 3] and margin == 0.0
    np.testing.assert_allclose(oracle.gate_dense(np.zeros(16), 4)[:4], 0.25, rtol=0)
    # selection order is by score, largest first
    idx, margin = oracle.topk(np.array([0.1, 0.5, 0.5, 0.9, -1.0]), 3)
    assert list(idx) == [3, 1, 2] and abs(margin - 0.4) < 1e-15


# ---------------------------------------------------------------------------
# Per-expert norm before mixing: the page's counterexample, through forward()
# ---------------------------------------------------------------------------

def test_norm_before_mix_counterexample():
    g = read_golden("norm_before_mix.txt")
    e1, e2 = np.array(g["e1"]), np.array(g["e2"])
    # Two ReLU experts whose outputs on x = (1,1) are e1 and e2; router weights zero -> tie -> weights 1/2.
    cfg = f32cfg(d=2, n=2, k=2, F=2, expert_norm="input_scaled")
    w1 = np.stack([np.eye(2), np.eye(2)]).astype(np.float32)
    w2 = np.stack([np.diag(e1), np.diag(e2)]).astype(np.float32)  # W2 @ relu(x) with x = (1,1)
    t = {"x": np.ones((1, 2), np.float32), "router_w": np.zeros((2, 2), np.float32), "w1": w1, "w2": w2,
         "gamma_ex": np.zeros(2, np.float32)}
    r = oracle.forward(cfg, t)
    np.testing.assert_allclose(r["w"][0], [0.5, 0.5])
    np.testing.assert_allclose(r["y"][0] ** 2, g["individual_sq"], rtol=1e-15)
    mixed = oracle.rms_centered(0.5 * e1 + 0.5 * e2, None, 0.0)
    np.testing.assert_allclose(mixed, np.array(g["mixed_num"]) / math.sqrt(g["mixed_den_sq"][0]), rtol=1e-15)
    assert np.abs(r["y"][0] - mixed).max() > 0.5   # the orders differ


# ---------------------------------------------------------------------------
# Experts: closed forms of SwiGLU wiring (gate rows first, then up rows)
# ---------------------------------------------------------------------------

def test_swiglu_identity_closed_form():
    # L = F = 4, no latent scaling: down = up = I, gate rows = I, up rows = 2I, W2 = I.
    D = 4
    cfg = dict(d=D, L=D, n=2, k=1, F=D, kind="swiglu3", act="f32", weights="f32", router_w="f32",
               in_norm="none", expert_norm="none", res_gate="linear", eps_in=0.0, eps_expert=0.0)
    I = np.eye(D, dtype=np.float32)
    w1 = np.stack([np.concatenate([I, 2 * I]), np.concatenate([I, 2 * I])])
    w2 = np.stack([I, I])
    x = np.array([[0.5, -1.25, 2.0, 0.0]], np.float32)
    gate = np.array([1.0, 0.5, 0.0, 0.25], np.float32)
    t = {"x": x, "router_w": np.zeros((2, D), np.float32), "down_w": I, "w1": w1, "w2": w2, "up_w": I, "gate": gate}
    r = oracle.forward(cfg, t)
    z = x[0].astype(np.float64)
    silu = z / (1 + np.exp(-z))
    np.testing.assert_allclose(r["y"][0], silu * (2 * z), rtol=1e-15, atol=1e-300)
    np.testing.assert_allclose(r["out"][0], z + gate * silu * (2 * z), rtol=1e-15)


def test_identical_experts_make_routing_irrelevant():
    # All experts equal and sum of weights 1: y equals that expert's normalised output for every routing.
    p = synthetic.small(T=6, d=32, L=16, F=16, n=6, k=3)
    prm = synthetic.layer_params(p)
    prm["w1"] = np.broadcast_to(prm["w1"][0], prm["w1"].shape).copy()
    prm["w2"] = np.broadcast_to(prm["w2"][0], prm["w2"].shape).copy()
    x = synthetic.inputs(p)
    cfg = p.cfg()
    r = oracle.forward(cfg, dict(prm, x=x))
    forced = np.tile(np.array([[5, 0, 2]], np.int32), (p.T, 1))
    r2 = oracle.forward(cfg, dict(prm, x=x), forced=forced)
    np.testing.assert_allclose(r["y"], r2["y"], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Brute force: an independent numpy evaluation of the whole layer
# ---------------------------------------------------------------------------

def _numpy_layer(cfg, t, act_round, aq=None):
    """Plain numpy matmuls over all experts with the dense gate vector.
    aq (optional): the quantizer applied to the inputs of the expert GEMMs."""
    x = t["x"].astype(np.float64)
    T = x.shape[0]
    if cfg["in_norm"] == "centered":
        u = (1 + t["gamma_in"].astype(np.float64)) * x / np.sqrt((x * x).mean(1, keepdims=True) + cfg["eps_in"])
        u = act_round(u)
    elif cfg["in_norm"] == "input_scaled":
        s = act_round((1 + t["gamma_in"].astype(np.float64)) * x)
        u = act_round(s / np.sqrt((s * s).mean(1, keepdims=True) + cfg["eps_in"]))
    else:
        u = x
    logits = (u @ t["router_w"].astype(np.float64).T).astype(np.float32)
    sigmoid = cfg.get("router_fn", "softmax") == "sigmoid"
    if sigmoid:
        v = (logits.astype(np.float64) * cfg.get("out_mult", 1.0)).astype(np.float32)
        basis = scipy.special.expit(v.astype(np.float64)).astype(np.float32)
    else:
        basis = logits
    score = basis + t["bias"] if "bias" in t else basis
    n, k, F = cfg["n"], cfg["k"], cfg["F"]
    G = np.zeros((T, n))
    for i in range(T):
        order = sorted(range(n), key=lambda e: (-float(score[i, e]), e))[:k]
        H = basis[i, order].astype(np.float64)
        if sigmoid:
            G[i, order] = H / (H.sum() + 1e-15) * cfg.get("routed_scale", 1.0)
        else:
            G[i, order] = scipy.special.softmax(H)
    z = u @ t["down_w"].astype(np.float64).T if cfg["L"] else u
    if cfg.get("latent_norm", "none") == "centered":
        z = (1 + t["gamma_lat"].astype(np.float64)) * z / np.sqrt((z * z).mean(1, keepdims=True)
                                                                 + cfg["eps_latent"])
    if aq is not None:
        z = aq(z)
    m = np.zeros_like(z)
    for e in range(n):
        W1 = t["w1"][e].astype(np.float64)
        if cfg["kind"] == "swiglu3":
            gg, vv = z @ W1[:F].T, z @ W1[F:].T
            a = gg * scipy.special.expit(gg) * vv
        else:
            a = np.maximum(z @ W1.T, 0)
        if aq is not None:
            a = aq(a)
        o = a @ t["w2"][e].astype(np.float64).T
        if cfg["expert_norm"] == "input_scaled":
            s = act_round((1 + t["gamma_ex"].astype(np.float64)) * o)
            o = s / np.sqrt((s * s).mean(1, keepdims=True) + cfg["eps_expert"])
        m += G[:, e:e + 1] * o
    y = m @ t["up_w"].astype(np.float64).T if cfg["L"] else m
    if cfg.get("out_norm", "none") == "input_scaled":
        s = act_round((1 + t["gamma_out"].astype(np.float64)) * y)
        y = s / np.sqrt((s * s).mean(1, keepdims=True) + cfg["eps_out"])
    g = t["gate"].astype(np.float64) if "gate" in t else None
    if cfg["res_gate"] == "linear":
        out = x + g * y
    elif cfg["res_gate"] == "muse":
        w = g / cfg.get("res_tau", 0.3)
        beta = scipy.special.expit(w)
        alpha = np.sqrt(np.maximum(scipy.special.expit(-w) * (1 + beta), cfg.get("res_floor", 1e-3)))
        out = alpha * x + beta * y
    else:
        out = y
    return G, y, out


@pytest.mark.parametrize("in_norm", ["none", "centered", "input_scaled"])
@pytest.mark.parametrize("bias", [False, True])
def test_bruteforce_latent_layer_f32(in_norm, bias):
    rng = np.random.default_rng(7)
    d, L, F, n, k, T = 24, 12, 10, 7, 3, 9
    cfg = dict(d=d, L=L, n=n, k=k, F=F, kind="swiglu3", act="f32", weights="f32", router_w="f32",
               in_norm=in_norm, expert_norm="input_scaled", res_gate="linear", eps_in=1e-5, eps_expert=1e-6)
    f = lambda *s: (rng.standard_normal(s) * 0.4).astype(np.float32)
    t = {"x": f(T, d) * 2, "router_w": f(n, d), "down_w": f(L, d), "w1": f(n, 2 * F, L), "w2": f(n, L, F),
         "up_w": f(d, L), "gamma_ex": f(L) * 0.1, "gamma_in": f(d) * 0.1,
         "gate": rng.uniform(0, 1, d).astype(np.float32)}
    if bias:
        t["bias"] = f(n)
    r = oracle.forward(cfg, t)
    rd = oracle.forward(cfg, t, dense=True)
    G, y, out = _numpy_layer(cfg, t, lambda v: v.astype(np.float32).astype(np.float64))
    for i in range(T):
        np.testing.assert_allclose(G[i, r["idx"][i]], r["w"][i], rtol=1e-13)
        assert (G[i] > 0).sum() == k
    np.testing.assert_allclose(r["y"], y, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["out"], out, rtol=1e-10, atol=1e-12)
    # sparse dispatch equals the dense sum over all n experts
    np.testing.assert_allclose(r["y"], rd["y"], rtol=1e-12, atol=1e-13)


def test_bruteforce_relu_layer_c0_shape():
    p = synthetic.PRESETS["c0"]
    prm = synthetic.layer_params(p)
    x = synthetic.inputs(p)[:16]
    t = dict(prm, x=x)
    cfg = p.cfg()
    r = oracle.forward(cfg, t)
    G, y, out = _numpy_layer(cfg, t, None)
    np.testing.assert_allclose(r["y"], y, rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(r["out"], r["y"])   # out = y: no residual gate
    rd = oracle.forward(cfg, t, dense=True)
    np.testing.assert_allclose(r["y"], rd["y"], rtol=1e-12, atol=1e-13)


def test_bruteforce_bf16_small_layer():
    # bf16 stored weights and activations; the rounding of I_gamma's scaled vector via torch.
    p = synthetic.small(T=5, d=64, L=32, F=32, n=8, k=2)
    t = dict(synthetic.layer_params(p), x=synthetic.inputs(p))
    cfg = p.cfg()
    r = oracle.forward(cfg, t)
    tf = {kk: (synthetic.bf16_to_f32(v) if v.dtype == np.uint16 else v) for kk, v in t.items()}
    bf = lambda v: torch.from_numpy(np.asarray(v, np.float64)).to(torch.bfloat16).to(torch.float64).numpy()
    G, y, out = _numpy_layer(cfg, tf, bf)
    np.testing.assert_allclose(r["y"], y, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(r["out"], out, rtol=1e-9, atol=1e-12)


def test_rows_are_independent():
    p = synthetic.small(T=10, d=64, L=32, F=32, n=8, k=2)
    t = dict(synthetic.layer_params(p), x=synthetic.inputs(p))
    cfg = p.cfg()
    full = oracle.forward(cfg, t)
    part = oracle.forward(cfg, t, tokens=np.array([7, 2, 9]))
    np.testing.assert_array_equal(part["y"], full["y"][[7, 2, 9]])
    np.testing.assert_array_equal(part["idx"], full["idx"][[7, 2, 9]])


# ---------------------------------------------------------------------------
# Permutation: invariants and a library sort
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,k,n", [(1, 1, 1), (37, 4, 16), (300, 8, 256), (64, 2, 8)])
def test_permutation_invariants(T, k, n):
    rng = np.random.default_rng(T + k + n)
    idx = np.stack([rng.choice(n, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    r = oracle.permute(idx, n)
    assert r["counts"].sum() == T * k
    np.testing.assert_array_equal(r["offsets"], np.concatenate([[0], np.cumsum(r["counts"])]))
    # a library stable sort by (expert, token)
    tt = np.repeat(np.arange(T), k)
    jj = np.tile(np.arange(k), T)
    order = np.lexsort((tt, idx.reshape(-1)))
    np.testing.assert_array_equal(r["perm_tok"], tt[order])
    np.testing.assert_array_equal(r["perm_slot"], jj[order])
    # inverse: pos[t, j] points back to (t, j)
    np.testing.assert_array_equal(r["perm_tok"][r["pos"]], np.repeat(np.arange(T)[:, None], k, 1))
    np.testing.assert_array_equal(r["perm_slot"][r["pos"]], np.tile(np.arange(k)[None, :], (T, 1)))


# ---------------------------------------------------------------------------
# MXFP4 decode: exhaustive against the OCP MX v1.0 E2M1 table
# ---------------------------------------------------------------------------

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


@pytest.mark.parametrize("E", [0, 1, 100, 120, 127, 130, 200, 254])
def test_mxfp4_decode_exhaustive(E):
    K = 32
    codes = np.array([c for c in range(16)] * 2, np.uint8)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    buf = np.concatenate([packed, np.array([E], np.uint8)])
    dec = oracle.decode_matrix(buf, "mxfp4", 1, K)[0]
    expect = np.array([E2M1[c] for c in codes]) * 2.0 ** (E - 127)
    np.testing.assert_array_equal(dec, expect)


def test_mxfp4_quantiser_round_trip_and_rne():
    # values on the grid times a power of two come back exactly; amax decides the scale
    rng = np.random.default_rng(5)
    rows = []
    for s in (-7, 0, 3):
        v = np.array([E2M1[c] for c in rng.integers(0, 16, 32)], np.float32)
        v[0] = 6.0  # amax 6 -> floor(log2 6) - 2 = 0 -> scale 2^0 relative
        rows.append(v * np.float32(2.0 ** s))
    v = np.stack(rows)
    buf = synthetic.mxfp4_quantize(v)
    np.testing.assert_array_equal(oracle.decode_matrix(buf, "mxfp4", 3, 32), v.astype(np.float64))
    # ties go to the even code: amax 4 -> scale 1 (floor(log2 4) - 2 = 0)
    w = np.zeros((1, 32), np.float32)
    w[0, :8] = [4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    dec = oracle.decode_matrix(synthetic.mxfp4_quantize(w), "mxfp4", 1, 32)[0]
    np.testing.assert_array_equal(dec[:8], [4.0, 0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0])
    # saturation: amax 7 -> scale 2^0 -> 7 saturates to 6
    w[0, 0] = 7.0
    assert oracle.decode_matrix(synthetic.mxfp4_quantize(w), "mxfp4", 1, 32)[0, 0] == 6.0


# ---------------------------------------------------------------------------
# Shapes: the parameter arithmetic of the 816B-A42B layer
# ---------------------------------------------------------------------------

def test_latent_layer_parameter_counts():
    p = synthetic.PRESETS["c1"]
    per_expert = 2 * p.F * p.L + p.L * p.F
    assert per_expert == 3 * 4096 ** 2 == 50_331_648
    total_experts = per_expert * p.n * 62
    assert abs(total_experts / 816e9 - 0.979) < 0.001          # "about 97%" of 816B
    assert abs(p.k * per_expert * 62 / 1e9 - 24.96) < 0.01    # about 25B active expert parameters
    # the two-matrix 8192->4096->8192 reading would exceed the total
    assert 2 * 8192 * 4096 * 256 * 62 > 816e9


def test_round_f16_matches_library_and_ties():
    rng = np.random.default_rng(2)
    vals = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-9, 5, 2000),
                           [1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 65504.0, 65519.0, 65520.0, 2 ** -25, 3 * 2 ** -25]])
    ours = np.array([oracle.round_f16(v) for v in vals])
    ref = torch.tensor(vals).to(torch.float16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)
    assert oracle.round_f16(1.0 + 2 ** -11) == 1.0 and oracle.round_f16(65520.0) == np.inf


# ---------------------------------------------------------------------------
# Sigmoid router (gates page, "Latent experts: normalization happens before
# the weighted sum": FP32 logits times output_multiplier, sigmoid, a
# selection-only correction bias, weights = kept sigmoids / (sum + 1e-15)
# times routed_scaling_factor; fact sheet: gating function sigmoid)
# ---------------------------------------------------------------------------

def _sig_layer(logits, k, **kw):
    n = len(logits)
    x, W = _router_layer(np.asarray(logits, np.float32))
    cfg = f32cfg(d=n, n=n, k=k, F=2, router_fn="sigmoid", **kw)
    t = {"x": x, "router_w": W, "w1": np.zeros((n, 2, n), np.float32), "w2": np.zeros((n, n, 2), np.float32)}
    return cfg, t


def test_sigmoid_router_closed_form():
    # logits 0, 1, -1, 2 times ln 3: sigmoids 1/2, 3/4, 1/4, 9/10 (sigma(m ln 3) = 3^m / (3^m + 1))
    cfg, t = _sig_layer([0, 1, -1, 2], 2, out_mult=math.log(3), routed_scale=2.0)
    sel, H = oracle.router_scores(cfg, [[0, 1, -1, 2]])
    np.testing.assert_allclose(H[0], [0.5, 0.75, 0.25, 0.9], rtol=1e-7)   # fp32 sigmoids
    np.testing.assert_array_equal(sel, H)                                  # no bias
    r = oracle.forward(cfg, t)
    assert list(r["idx"][0]) == [3, 1]
    np.testing.assert_allclose(r["w"][0], [2 * 0.9 / 1.65, 2 * 0.75 / 1.65], rtol=1e-7)   # 12/11, 10/11
    # a bias of +1 on expert 2 moves it into the selection (1.25 > 0.9 > 0.75) but
    # its weight still uses its own sigmoid 1/4: weights 2 * (1/4, 9/10) / (23/20)
    t["bias"] = np.array([0, 0, 1, 0], np.float32)
    r = oracle.forward(cfg, t)
    assert list(r["idx"][0]) == [2, 3]
    np.testing.assert_allclose(r["w"][0], [10 / 23, 36 / 23], rtol=1e-7)
    assert abs(r["margin"][0] - 0.15) < 1e-6   # 0.9 - 0.75


def test_sigmoid_router_saturation_and_underflow():
    # every kept sigmoid rounds to 0 in fp32: the 1e-15 keeps the weights at exactly 0
    cfg, t = _sig_layer([-200, -300, -150, -180], 2, routed_scale=1.0)
    r = oracle.forward(cfg, t)
    assert list(r["idx"][0]) == [0, 1]          # all scores 0: ties to the lower id
    np.testing.assert_array_equal(r["w"][0], [0.0, 0.0])
    # every sigmoid rounds to 1: equal weights rsf / (k + 1e-15)
    cfg, t = _sig_layer([40, 50, 60, 70], 3, routed_scale=2.5)
    r = oracle.forward(cfg, t)
    assert list(r["idx"][0]) == [0, 1, 2]
    np.testing.assert_allclose(r["w"][0], 2.5 / 3, rtol=1e-15)


@pytest.mark.parametrize("n,k", [(16, 4), (256, 8)])
def test_sigmoid_selection_is_monotone_and_weights_renormalise(n, k):
    rng = np.random.default_rng(n + k)
    for _ in range(20):
        lg = (rng.standard_normal(n) * 2).astype(np.float32)
        cs = f32cfg(n=n, k=k, router_fn="sigmoid", out_mult=0.7, routed_scale=1.5)
        sel, H = oracle.router_scores(cs, lg)
        idx, _ = oracle.topk(sel[0], k)
        # the sigmoid is increasing: without a bias it keeps the k largest logits
        idx_l, _ = oracle.topk(lg.astype(np.float64), k)
        assert set(idx) == set(idx_l)
        w = oracle.router_weights(cs, H[0], idx)
        assert (w > 0).all() and abs(w.sum() - 1.5) < 1e-12
        # k = n: every sigmoid, normalised by their total
        wn = oracle.router_weights(cs, H[0], np.arange(n, dtype=np.int32))
        np.testing.assert_allclose(wn, 1.5 * H[0] / H[0].sum(), rtol=1e-13)


# ---------------------------------------------------------------------------
# Residual gate (gates page, "Residual gates: derive the advertised
# intuition carefully"; fact sheet residual design)
# ---------------------------------------------------------------------------

def test_residual_gate_identity_and_floor():
    g = np.linspace(-2.2, 2.2, 89)
    al, be = oracle.muse_gate_coeffs(g, 0.3, 1e-3)
    # sigma(-w) = 1 - beta, so while the floor is inactive alpha^2 = 1 - beta^2
    np.testing.assert_allclose(al ** 2 + be ** 2, 1.0, rtol=0, atol=4e-16)
    assert (np.diff(be) > 0).all() and (np.diff(al) < 0).all()
    np.testing.assert_allclose(be, 1 / (1 + np.exp(-g / 0.3)), rtol=1e-15)
    # the floor: sigma(-w)(1 + beta) < 1e-3 once g / 0.3 > ln(2000) (g > 2.28)
    al, be = oracle.muse_gate_coeffs([2.27, 2.29, 3.0, 30.0], 0.3, 1e-3)
    assert al[0] > math.sqrt(1e-3)
    np.testing.assert_array_equal(al[1:], math.sqrt(1e-3))
    assert al[3] ** 2 + be[3] ** 2 > 1.0009      # clamped: the identity no longer holds
    # a temperature of 0.3 against 1: the same g gives a sharper beta
    _, b1 = oracle.muse_gate_coeffs([0.6], 1.0, 1e-3)
    _, b3 = oracle.muse_gate_coeffs([0.6], 0.3, 1e-3)
    assert b3[0] > b1[0] > 0.5


def _gate_layer(W2, gate_g):
    """d = 2 ReLU layer, one expert with W1 = I: y = W2 relu(x); Muse gate g."""
    cfg = f32cfg(d=2, n=1, k=1, F=2, res_gate="muse", res_tau=0.3, res_floor=1e-3)
    t = {"x": np.array([[1.0, 0.0]], np.float32), "router_w": np.zeros((1, 2), np.float32),
         "w1": np.eye(2, dtype=np.float32)[None], "w2": np.asarray(W2, np.float32)[None],
         "gate": np.full(2, gate_g, np.float32)}
    return oracle.forward(cfg, t)


def test_residual_gate_geometry_worked_example():
    gd = read_golden("residual_gate_geometry.txt")
    al, be = oracle.muse_gate_coeffs([0.0], gd["tau"][0], gd["floor"][0])
    assert be[0] == gd["beta"][0]
    np.testing.assert_allclose(al[0] ** 2, gd["alpha_sq"][0], rtol=1e-15)
    # equal-norm residual r = (1, 0) and branch b = W2 relu(r): orthogonal, aligned, opposite
    cases = {"orthogonal": [[0, 0], [1, 0]], "aligned": [[1, 0], [0, 1]], "opposite": [[-1, 0], [0, -1]]}
    exact = {"orthogonal": 1.0, "aligned": 1 + math.sqrt(3) / 2, "opposite": 1 - math.sqrt(3) / 2}
    for name, W2 in cases.items():
        r = _gate_layer(W2, 0.0)
        f = float((r["out"][0] ** 2).sum())
        assert abs(f - gd[name][0]) < 5e-4, name          # the page's three places
        np.testing.assert_allclose(f, exact[name], rtol=1e-14)


def test_muse_gate_wiring_against_linear_gate():
    # g = 0 everywhere: out = (sqrt 3 / 2) x + y / 2, where x + y is the linear gate's output with g = 1
    p = synthetic.small(T=6, d=64, L=32, F=32, n=8, k=2, out_norm="input_scaled", latent_norm="centered")
    prm = synthetic.layer_params(p)
    t = dict(prm, x=synthetic.inputs(p))
    t["gate"] = np.ones(p.d, np.float32)
    r_lin = oracle.forward(p.cfg(), t)
    cfg = dict(p.cfg(), res_gate="muse")
    t["gate"] = np.zeros(p.d, np.float32)
    r_m = oracle.forward(cfg, t)
    x = synthetic.bf16_to_f32(t["x"]).astype(np.float64)
    np.testing.assert_allclose(r_m["y"], r_lin["y"], rtol=0, atol=0)
    np.testing.assert_allclose(r_m["out"], math.sqrt(3) / 2 * x + 0.5 * (r_lin["out"] - x), rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------------------
# Latent pre-norm z = C_pre(P_down u) and the FFN output norm (gates page,
# "Latent experts ..." and "The complete layer has two separately normalized
# residual updates")
# ---------------------------------------------------------------------------

def _f32_latent(**kw):
    rng = np.random.default_rng(21)
    d, L, F, n, k, T = 16, 8, 8, 5, 2, 7
    cfg = dict(d=d, L=L, n=n, k=k, F=F, kind="swiglu3", act="f32", weights="f32", router_w="f32",
               in_norm="none", expert_norm="input_scaled", res_gate="none", eps_in=0.0, eps_expert=1e-6,
               eps_latent=0.0, eps_out=0.0)
    cfg.update(kw)
    f = lambda *s: (rng.standard_normal(s) * 0.5).astype(np.float32)
    t = {"x": f(T, d), "router_w": f(n, d), "down_w": f(L, d), "w1": f(n, 2 * F, L), "w2": f(n, L, F),
         "up_w": f(d, L), "gamma_ex": f(L) * 0.1, "gamma_lat": f(L) * 0.2, "gamma_out": f(d) * 0.2,
         "gate": rng.uniform(-3, 3, d).astype(np.float32)}
    return cfg, t


def test_latent_prenorm_removes_the_scale_of_the_down_projection():
    cfg, t = _f32_latent(latent_norm="centered")
    r = oracle.forward(cfg, t)
    t4 = dict(t, down_w=t["down_w"] * 4)            # exact in fp32: C(4z) = C(z) with eps = 0
    np.testing.assert_allclose(oracle.forward(cfg, t4)["y"], r["y"], rtol=1e-13, atol=1e-15)
    cfg0 = dict(cfg, latent_norm="none")           # without it the SwiGLU sees a 4x larger z
    assert np.abs(oracle.forward(cfg0, t4)["y"] - oracle.forward(cfg0, t)["y"]).max() > 1e-3


def test_output_norm_scale_invariance_and_unit_rms():
    cfg, t = _f32_latent(out_norm="input_scaled")
    r = oracle.forward(cfg, t)
    np.testing.assert_allclose(np.sqrt((r["y"] ** 2).mean(1)), 1.0, rtol=1e-13)   # eps = 0: unit RMS
    t2 = dict(t, up_w=t["up_w"] * 2)
    np.testing.assert_array_equal(oracle.forward(cfg, t2)["y"], r["y"])          # powers of two are exact
    # I_gamma, not C_gamma: the gain enters before the denominator
    cc = oracle.forward(dict(cfg, out_norm="centered"), t)
    assert np.abs(cc["y"] - r["y"]).max() > 1e-3


@pytest.mark.parametrize("bias", [False, True])
def test_bruteforce_muse_layer_f32(bias):
    cfg, t = _f32_latent(in_norm="centered", latent_norm="centered", out_norm="input_scaled", res_gate="muse",
                         router_fn="sigmoid", out_mult=0.8, routed_scale=1.7, eps_in=1e-5, eps_latent=1e-5,
                         eps_out=1e-5)
    t["gamma_in"] = (np.random.default_rng(3).standard_normal(cfg["d"]) * 0.1).astype(np.float32)
    if bias:
        t["bias"] = (np.random.default_rng(4).standard_normal(cfg["n"]) * 0.3).astype(np.float32)
    r = oracle.forward(cfg, t)
    rd = oracle.forward(cfg, t, dense=True)
    G, y, out = _numpy_layer(cfg, t, lambda v: v.astype(np.float32).astype(np.float64))
    for i in range(t["x"].shape[0]):
        np.testing.assert_allclose(G[i, r["idx"][i]], r["w"][i], rtol=1e-13)
        assert (G[i] > 0).sum() == cfg["k"]
    np.testing.assert_allclose(r["y"], y, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["out"], out, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["y"], rd["y"], rtol=1e-12, atol=1e-13)


def test_bruteforce_muse_bf16_small_layer():
    p = synthetic.muse("mini", T=5, d=64, L=32, F=32, n=8, k=2, layer_seed=11)
    t = dict(synthetic.layer_params(p), x=synthetic.inputs(p))
    cfg = p.cfg()
    r = oracle.forward(cfg, t)
    tf = {kk: (synthetic.bf16_to_f32(v) if v.dtype == np.uint16 else v) for kk, v in t.items()}
    bf = lambda v: torch.from_numpy(np.asarray(v, np.float64)).to(torch.bfloat16).to(torch.float64).numpy()
    G, y, out = _numpy_layer(cfg, tf, bf)
    np.testing.assert_allclose(r["y"], y, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(r["out"], out, rtol=1e-9, atol=1e-12)


# ---------------------------------------------------------------------------
# MXFP8 activations (OCP MX v1.0: E4M3 elements, one power-of-two scale per
# 32 values along K, X = floor(log2 amax) - 8, round to nearest even,
# magnitudes past 448 clamped)
# ---------------------------------------------------------------------------

def _e4m3_library(v):
    """torch's float8_e4m3fn conversion (round to nearest even; it returns
    NaN past 464 instead of clamping, so clamp first)."""
    v = np.clip(np.asarray(v, np.float64), -448.0, 448.0)
    return torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_mxfp8_element_grid_is_e4m3():
    # a dense sweep of one block scale: the distinct outputs are exactly the 127 non-negative finite
    # E4M3 values (the OCP FP8 E4M3 format has 8 per binade from 2^-6 to 2^8, subnormals of 2^-9)
    v = np.linspace(0, 448, 32 * 20000)
    v[::32] = 448.0  # every block's max is 448: X = floor(log2 448) - 8 = 0
    q, X = oracle.mxfp8_quantize(v)
    assert (X == 0).all()
    vals = np.unique(q)
    assert len(vals) == 127 and vals[0] == 0 and vals[1] == 2.0 ** -9 and vals[-1] == 448.0
    for e in range(-6, 9):
        inb = vals[(vals >= 2.0 ** e) & (vals < 2.0 ** (e + 1))]
        assert len(inb) == (7 if e == 8 else 8)


def test_mxfp8_matches_library_rounding_and_ties():
    rng = np.random.default_rng(3)
    # random values whose block max is 448 (scale 1), midpoints of the E4M3 grid included
    v = rng.uniform(-448, 448, (2000, 32))
    v[:, 0] = 448.0
    mids = np.array([1 + 1 / 16, 1.1875, 2.0 ** -9 * 1.5, 2.0 ** -9 * 0.5, 300.0, 272.0, 304.0, -1.0625])
    v[:8, 1:1 + len(mids)] = mids
    q, X = oracle.mxfp8_quantize(v)
    assert (X == 0).all()
    np.testing.assert_array_equal(q, _e4m3_library(v))
    # ties go to the even mantissa: 1 + 1/16 -> 1, 1.1875 -> 1.25, 1.5 * 2^-9 -> 2^-8, 0.5 * 2^-9 -> 0
    np.testing.assert_array_equal(q[0, 1:6], [1.0, 1.25, 2.0 ** -8, 0.0, 288.0])


def test_mxfp8_shared_scale_closed_form():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((500, 64)) * np.exp2(rng.integers(-20, 12, (500, 1)))
    q, X = oracle.mxfp8_quantize(v)
    blocks = v.reshape(500, 2, 32)
    amax = np.abs(blocks).max(axis=2)
    m, e = np.frexp(amax)          # amax = m * 2^e, m in [0.5, 1): floor(log2 amax) = e - 1
    np.testing.assert_array_equal(X, e - 1 - 8)
    # the element values are the library's E4M3 rounding of v / 2^X, and the block max lands in [256, 448]
    sc = np.exp2(X.astype(np.float64))[:, :, None]
    ref = _e4m3_library(blocks / sc) * sc
    np.testing.assert_array_equal(q.reshape(500, 2, 32), ref)
    qm = np.abs(q.reshape(500, 2, 32)).max(axis=2) / sc[:, :, 0]
    assert ((qm >= 256) & (qm <= 448)).all()
    # below 448 * 2^X an element moves by at most half an E4M3 spacing (2^-4 of its magnitude, or half the
    # subnormal spacing 2^(X-10)); at or past it, it clamps to 448 * 2^X
    Xe = np.exp2(X.repeat(32, axis=1).astype(np.float64))
    inside = np.abs(v) < 448 * Xe
    assert (np.abs(q - v)[inside] <= np.maximum(np.abs(v) * 2.0 ** -4, Xe * 2.0 ** -10)[inside]).all()
    np.testing.assert_array_equal(np.abs(q)[~inside], 448 * Xe[~inside])


def test_mxfp8_zero_block_and_idempotence():
    v = np.zeros((3, 32))
    v[1, 5] = -3.0
    q, X = oracle.mxfp8_quantize(v)
    assert X[0, 0] == -127 and (q[0] == 0).all()
    assert X[1, 0] == 1 - 8 and q[1, 5] == -3.0 and (np.delete(q[1], 5) == 0).all()
    rng = np.random.default_rng(5)
    w = rng.standard_normal((100, 96))
    q1, X1 = oracle.mxfp8_quantize(w)
    q2, X2 = oracle.mxfp8_quantize(q1)   # already on the grid: unchanged
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(X1, X2)


def _mx_act(interm):
    """An independent statement of the activation quantizer: the stored
    intermediate (torch's fp16 or bf16 rounding), then the library's E4M3
    rounding on the shared scale of each 32-block."""
    tdt = torch.float16 if interm == "f16" else torch.bfloat16

    def q(a):
        a = torch.from_numpy(np.asarray(a, np.float64)).to(tdt).to(torch.float64).numpy()
        b = a.reshape(a.shape[:-1] + (a.shape[-1] // 32, 32))
        amax = np.abs(b).max(axis=-1, keepdims=True)
        e = np.frexp(np.where(amax > 0, amax, 1.0))[1]
        sc = np.exp2((e - 1 - 8).astype(np.float64))
        out = np.where(amax > 0, _e4m3_library(b / sc) * sc, 0.0)
        return out.reshape(a.shape)
    return q


@pytest.mark.parametrize("interm", ["f16", "bf16"])
def test_bruteforce_mxfp8_activation_layer(interm):
    # the quantized-activation mode through the whole layer against the numpy brute force with the
    # quantizer applied where the expert GEMMs read: the latent z and the SwiGLU output
    p = synthetic.small(T=7, d=128, L=64, F=64, n=8, k=2, weights="mxfp4")
    t = dict(synthetic.layer_params(p), x=synthetic.inputs(p))
    cfg = dict(p.cfg(), act_quant="mxfp8", interm=interm)
    r = oracle.forward(cfg, t)
    tf = {kk: (synthetic.bf16_to_f32(v) if v.dtype == np.uint16 else v) for kk, v in t.items()}
    for key, rows, K in (("down_w", p.L, p.d), ("up_w", p.d, p.L), ("w1", p.n * 2 * p.F, p.L),
                         ("w2", p.n * p.L, p.F)):
        dec = oracle.decode_matrix(t[key], "mxfp4", rows, K)
        tf[key] = dec.reshape((p.n, 2 * p.F, p.L) if key == "w1" else (p.n, p.L, p.F) if key == "w2" else (rows, K))
    bf = lambda v: torch.from_numpy(np.asarray(v, np.float64)).to(torch.bfloat16).to(torch.float64).numpy()
    G, y, out = _numpy_layer(cfg, tf, bf, aq=_mx_act(interm))
    np.testing.assert_allclose(r["y"], y, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(r["out"], out, rtol=1e-9, atol=1e-12)
    # the quantization is not a no-op: without it the layer differs
    r0 = oracle.forward(dict(cfg, act_quant="none"), t)
    assert np.abs(r0["y"] - r["y"]).max() > 1e-3 * np.abs(r["y"]).max()


@pytest.mark.parametrize("E", [127, 120, 131])
def test_mxfp8_decode_exhaustive(E):
    # every E4M3 code against the library's float8_e4m3fn value, times the block scale 2^(E-127)
    codes = np.arange(256, dtype=np.uint8)
    buf = np.concatenate([codes, np.full(256 // 32, E, np.uint8)])
    got = oracle.decode_matrix(buf, "mxfp8", 1, 256)[0]
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy() * 2.0 ** (E - 127)
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.isnan(got[nan]).all()
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def test_mxfp8_quantize_then_decode_round_trip():
    # codes made from the quantizer's own values (library encoding) decode back to them exactly
    rng = np.random.default_rng(6)
    v = rng.standard_normal((3, 64)) * np.exp2(rng.integers(-10, 10, (3, 1)))
    q, X = oracle.mxfp8_quantize(v)
    sc = np.exp2(X.repeat(32, axis=1).astype(np.float64))
    codes = torch.from_numpy(q / sc).to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(-1)
    buf = np.concatenate([codes, (X + 127).astype(np.uint8).reshape(-1)])
    np.testing.assert_array_equal(oracle.decode_matrix(buf, "mxfp8", 3, 64), q)


def test_forced_expert_input():
    # the expert-space input given instead of computed: its own z reproduces the forward exactly; z = 0 gives
    # SwiGLU(0) = 0 in every expert, so the branch output is 0 and out = x (the linear gate)
    p = synthetic.small(T=5, d=64, L=32, F=32, n=8, k=2, weights="mxfp4")
    t = dict(synthetic.layer_params(p), x=synthetic.inputs(p))
    for aq in ("none", "mxfp8"):
        cfg = dict(p.cfg(), act_quant=aq)
        r = oracle.forward(cfg, t, want_z=True)
        r2 = oracle.forward(cfg, t, forced_z=r["z"])
        np.testing.assert_array_equal(r2["out"], r["out"])
        r0 = oracle.forward(cfg, t, forced_z=np.zeros_like(r["z"]))
        assert (r0["y"] == 0).all()
        np.testing.assert_array_equal(r0["out"], synthetic.bf16_to_f32(t["x"]).astype(np.float64))
    # under MXFP8 the z the experts read is on the E4M3 grid of its blocks
    zq, _ = oracle.mxfp8_quantize(r["z"])
    np.testing.assert_array_equal(zq, r["z"])
    # the hidden activations given instead of computed: its own reproduce the forward; zeros give o = 0 in
    # every selected expert, so again y = 0
    ra = oracle.forward(cfg, t, want_a=True)
    aq, _ = oracle.mxfp8_quantize(ra["a"])
    np.testing.assert_array_equal(aq, ra["a"])
    np.testing.assert_array_equal(oracle.forward(cfg, t, forced_a=ra["a"])["out"], ra["out"])
    assert (oracle.forward(cfg, t, forced_a=np.zeros_like(ra["a"]))["y"] == 0).all()
