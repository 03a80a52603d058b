"""Helpers of the GPU parity tests: move seeded host inputs to the device,
run the HIP layer through the C ABI, and compare with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import sparse_mixture_experts_router_amd as moe
import synthetic
from conftest import preset_desc

MARGIN_EXCLUDE = 1e-4
TOL = {"f32": 1e-5, "bf16": 2e-2, "mxfp4": 5e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def desc_of(p: synthetic.Preset, T: int | None = None):
    return preset_desc(p, T)


class DeviceLayer:
    """Layer parameters of a preset on the device (and their host copies)."""

    def __init__(self, p: synthetic.Preset, host: dict | None = None):
        self.p = p
        self.host = host if host is not None else synthetic.layer_params(p)
        self.dev = {}
        for k_, v in self.host.items():
            if "@" in k_:
                continue
            self.dev[k_] = to_dev(v)

    def gains(self):
        return {"router_bias": self.dev.get("bias"), "gamma_in": self.dev.get("gamma_in"),
                "gamma_expert": self.dev.get("gamma_ex"), "res_gate": self.dev.get("gate"),
                "gamma_latent": self.dev.get("gamma_lat"), "gamma_out": self.dev.get("gamma_out")}


def run(layer: DeviceLayer, x: np.ndarray, dbg: bool = True, workspace=None, stages: bool = True):
    p = layer.p
    T = x.shape[0]
    desc = desc_of(p, T)
    xd = to_dev(x)
    out = torch.empty((T, p.d), dtype=torch.float32, device="cuda")
    D = None
    if dbg:
        D = {"topk_idx": torch.empty((T, p.k), dtype=torch.int32, device="cuda"),
             "topk_w": torch.empty((T, p.k), dtype=torch.float32, device="cuda"),
             "expert_counts": torch.empty(p.n, dtype=torch.int32, device="cuda"),
             "expert_offsets": torch.empty(p.n + 1, dtype=torch.int32, device="cuda"),
             "perm_tok": torch.empty(T * p.k, dtype=torch.int32, device="cuda"),
             "perm_slot": torch.empty(T * p.k, dtype=torch.int32, device="cuda"),
             "y": torch.empty((T, p.d), dtype=torch.float32, device="cuda"),
             "pos": torch.empty((T, p.k), dtype=torch.int32, device="cuda"),
             "logits": torch.empty((T, p.n), dtype=torch.float32, device="cuda"),
             "u": torch.empty((T, p.d), dtype=torch.int16 if p.act == "bf16" else torch.float32, device="cuda")}
        if stages and p.act == "bf16":
            TK = T * p.k
            D.update({"z": torch.empty((T, p.L), dtype=torch.int16, device="cuda"),
                      "act": torch.empty((TK, p.F), dtype=torch.int16, device="cuda"),
                      "S": torch.empty((TK, p.L), dtype=torch.int16, device="cuda"),
                      "ssq": torch.empty((TK, p.L // 16), dtype=torch.float32, device="cuda"),
                      "m": torch.empty((T, p.L), dtype=torch.int16, device="cuda")})
            if p.act_quant == "mxfp8":
                D.update({"zq": torch.empty(T * p.L * 33 // 32, dtype=torch.uint8, device="cuda"),
                          "actq": torch.empty(TK * p.F * 33 // 32, dtype=torch.uint8, device="cuda")})
    dv = layer.dev
    moe.moe_layer_forward(desc, xd, dv["router_w"], dv.get("down_w"), dv["w1"], dv["w2"], dv.get("up_w"),
                          layer.gains(), out, workspace=workspace, dbg=D)
    torch.cuda.synchronize()
    res = {"out": out.cpu().numpy()}
    if dbg:
        for k_, v in D.items():
            a = v.cpu().numpy()
            res[k_] = a.view(np.uint16) if a.dtype == np.int16 else a
    return res


def oracle_cfg(p: synthetic.Preset) -> dict:
    return p.cfg()


def gate_weight_atol(p) -> float:
    """Tolerance of the gate weights.  Without an input norm both sides see
    the same stored u and their fp32 logits differ only by accumulation
    order (~1e-6), so 2e-5.  With an input norm, u is itself a bf16 rounding
    of a value the GPU computes in fp32 and the oracle in fp64: a few
    elements land one bf16 ulp (2^-8 relative) apart, shifting a logit by
    about sqrt(#flips) * 2^-8 * |u| * std(W) (~3e-4 for 1% flips at the
    tested shapes, 5 sigma ~1.5e-3 at d=8192) and a softmax weight by at most
    half of that, so 1e-3.  This end-to-end bar is not the only weight check:
    check_router_stage grades the weights to 2e-6 against the oracle applied
    to the device's own logits."""
    return 1e-3 if (p.act == "bf16" and p.in_norm != "none") else 2e-5


def check_router_stage(p, host, gpu, label="", known=None):
    """Router and top-k stage on every token of the batch, each against the
    oracle applied to the device's own stage input:
      logits: the oracle's router (fp64 dot products rounded to fp32) on the
              device's u, to 1e-4;
      experts: the oracle's top-k of the device's own fp32 logits, bit-exact
              on every token for the softmax router (both sides form the same
              fp32 scores l + b and break ties to the lower id); for the
              sigmoid router (device and oracle sigmoids may sit one fp32 ulp
              apart) on tokens whose k-th/(k+1)-th gap is >= 1e-6, in order
              where every adjacent gap of the top k+1 is;
      weights: the oracle's weights of the device's own logits and experts,
              to 2e-6 (times the routed scale).
    known: optional (logits, same) — the oracle's logits of every token from
    its own u, and which tokens' device u equals that u bit for bit; those
    logits are reused instead of routing the same input again."""
    cfg = dict(oracle_cfg(p), in_norm="none")
    u = gpu["u"]
    lg = gpu["logits"]
    T = lg.shape[0]
    ref = np.empty_like(lg)
    todo = np.arange(T)
    if known is not None:
        ref[known[1]] = known[0][known[1]]
        todo = np.flatnonzero(~known[1])
    for a in range(0, len(todo), 2048):  # oracle router on the device's branch input, in row blocks
        rows = todo[a:a + 2048]
        ref[rows] = oracle.forward(cfg, dict(host, x=u), tokens=rows, want_outputs=False)["logits"]
    dl = float(np.abs(lg - ref).max())
    sel, H = oracle.router_scores(cfg, lg, host.get("bias"))
    gidx = gpu["topk_idx"]
    sig = p.router_fn == "sigmoid"
    gap = 1e-6 if sig else 0.0
    bad_set, bad_order, nex = [], [], 0
    for t in range(T):
        ridx, margin = oracle.topk(sel[t], p.k)
        if p.k < p.n and margin < gap:
            nex += 1
            continue
        if set(ridx) != set(gidx[t]):
            bad_set.append(t)
        elif (ridx != gidx[t]).any():
            top = np.sort(sel[t])[::-1][:p.k + 1]
            if not sig or (np.diff(-top) >= gap).all():
                bad_order.append(t)
    wref = np.stack([oracle.router_weights(cfg, H[t], gidx[t]) for t in range(T)])
    dw = float(np.abs(gpu["topk_w"] - wref).max())
    say("  stage router/top-k %s: max|dlogit| %.3g, tokens %d (excluded %d), set mismatches %d, order "
        "mismatches %d, max|dw| %.3g" % (label, dl, T, nex, len(bad_set), len(bad_order), dw))
    assert dl <= 1e-4, "%s router logits %.3g from the oracle on the device's u" % (label, dl)
    assert not bad_set, "%s top-k sets differ from the oracle's on the device logits at %s" % (label, bad_set[:10])
    assert not bad_order, "%s top-k order differs at %s" % (label, bad_order[:10])
    assert dw <= 2e-6 * max(1.0, abs(p.routed_scale)), "%s gate weights %.3g" % (label, dw)


def check_input_norm(p, host, x, gpu, label="", u_orc=None):
    """The device's u = input norm of x on every token against the oracle's
    (fp64, rounded to bf16): equal except one-ulp flips on <= 0.5% of the
    elements (an fp32 and an fp64 value straddling a bf16 rounding
    boundary).  The input-scaled form rounds twice (s = bf16((1 + gamma) x),
    then u = bf16(s / rms(s))): where the device's s lands one ulp from the
    oracle's (its fp32 gain 1 + gamma and fp32 product round before the bf16
    step), u moves by one ulp of s and rounds again, so up to two ulps of u."""
    if p.in_norm == "none" or p.act != "bf16":
        return
    T = x.shape[0]
    nflip, nbad = 0, 0
    t = dict(host, x=x)
    for a in range(0, T, 1024):
        rows = np.arange(a, min(T, a + 1024))
        ur = oracle.branch_input(oracle_cfg(p), t, rows) if u_orc is None else u_orc[rows]
        d = np.abs(bf16f(gpu["u"][rows]) - ur)
        nflip += int((d > 0).sum())
        nbad += int((d > (2.01 if p.in_norm == "input_scaled" else 1.01) * ulp_bf16(ur)).sum())
    frac = nflip / float(T * p.d)
    say("  stage in_norm %s: %d rows, differing %.4f%%, beyond the ulp bound %d" % (label, T, 100 * frac, nbad))
    assert nbad == 0, "%s input norm: %d elements beyond the bf16 ulp bound" % (label, nbad)
    assert frac <= FLIP_FRACTION, "%s input norm: %.3g of elements differ" % (label, frac)


def check_routing(p, host, x, gpu, tokens, label="", u_orc=None):
    """Routing of rows `tokens`: expert sets bit-exact where the oracle's
    k-th/(k+1)-th score margin is >= 1e-4, order bit-exact where every
    adjacent gap of the top k+1 scores is >= 1e-4; gate weights to 2e-5.
    With an input norm, a token whose device u differs from the oracle's
    (one-bf16-ulp flips of the norm, graded by check_input_norm) routes on
    different fp32 logits; such tokens are left to check_router_stage,
    which routes the device's own u and logits bit-exactly."""
    t = dict(host)
    t["x"] = x
    r = oracle.forward(oracle_cfg(p), t, tokens=tokens, want_outputs=False)
    gidx = gpu["topk_idx"][tokens]
    s = oracle.router_scores(oracle_cfg(p), r["logits"], host.get("bias"))[0]   # selection scores
    clean = r["margin"] >= MARGIN_EXCLUDE
    same_u = np.ones(len(tokens), bool)
    wtol = gate_weight_atol(p)
    if p.in_norm != "none" and p.act == "bf16" and "u" in gpu:
        wtol = 2e-5  # tokens whose u differs are graded on the device's u instead
        for a in range(0, len(tokens), 1024):
            rows = np.asarray(tokens)[a:a + 1024]
            uo = oracle.branch_input(oracle_cfg(p), t, rows) if u_orc is None else u_orc[rows]
            same_u[a:a + 1024] = (bf16f(gpu["u"][rows]) == uo).all(axis=1)
        say("  routing %s: %d tokens whose device u has a one-ulp flip are graded on the device's u" % (
            label, int((~same_u).sum())))
        clean &= same_u
    if p.k < p.n:
        srt = -np.sort(-s.astype(np.float64), axis=1)[:, :p.k + 1]
        ordered = clean & ((srt[:, :-1] - srt[:, 1:]) >= MARGIN_EXCLUDE).all(axis=1)
    else:
        ordered = clean
    set_ok = np.array([set(gidx[i]) == set(r["idx"][i]) for i in range(len(tokens))])
    bad = np.flatnonzero(clean & ~set_ok)
    assert bad.size == 0, "%s routing sets differ at tokens %s" % (label, tokens[bad][:10])
    order_bad = np.flatnonzero(ordered & ~(gidx == r["idx"]).all(axis=1))
    assert order_bad.size == 0, "%s routing order differs at tokens %s" % (label, tokens[order_bad][:10])
    same = (gidx == r["idx"]).all(axis=1) & same_u
    np.testing.assert_allclose(gpu["topk_w"][tokens][same], r["w"][same], rtol=0, atol=wtol,
                               err_msg=label + " gate weights")
    return int((~clean).sum()), r["logits"], same_u


# The oracle's bf16-dataflow mode (z, the SwiGLU output and m rounded to
# bf16 where the device stores them) is reported beside the exact oracle.  It
# is not a tighter bar: a single one-ulp flip upstream (an fp32 and an fp64
# sum of the same products straddling a bf16 boundary) shifts every later
# value of that token slightly and re-draws a few percent of its later
# roundings, so whole-layer agreement with the dataflow oracle is of the order
# of the bf16 rounding noise itself.  The per-stage checks below (check_stages)
# are the tight ones.
TOL_DATAFLOW = {"f32": 1e-5, "bf16": 2e-2, "mxfp4": 5e-2}
DATAFLOW_TOKENS = 32

# The FFN output norm stores s = bf16((1 + gamma) y) (the input-scaled form
# rounds it there by definition; the output-scaled form is stored that way
# on the device).  Device and oracle reach y along different fp32 / fp64
# paths, so an element of s can land one bf16 ulp apart, which moves b by
# ulp(s) * inv: up to 2^-7 of |b|, about 1.6% of RMS(b) for the largest
# elements of a row, more than the bf16 tolerance leaves.  Such an element
# is allowed one ulp of s (times its gate coefficient in out); at most
# FLIP_OUT_FRACTION of the outputs may exceed the plain tolerance.
FLIP_OUT_FRACTION = 1e-2


def output_norm_allowance(p, host: dict, ypre: np.ndarray):
    """Per-element allowance (y, out) for the output norm's bf16 step."""
    if p.out_norm == "none":
        return 0.0, 0.0
    gam = 1.0 + host["gamma_out"].astype(np.float64)
    s_ref = round_bf16(gam * ypre)
    base = s_ref if p.out_norm == "input_scaled" else ypre
    inv = 1.0 / np.sqrt((base * base).mean(1, keepdims=True) + p.eps_out)
    allow_y = 1.01 * ulp_bf16(s_ref) * inv
    if p.res_gate == "linear":
        coef = np.abs(host["gate"].astype(np.float64))
    elif p.res_gate == "muse":
        coef = 1.0 / (1.0 + np.exp(-host["gate"].astype(np.float64) / p.res_tau))
    else:
        coef = 1.0
    return allow_y, allow_y * coef


def compare(p: synthetic.Preset, host: dict, x: np.ndarray, gpu: dict, tokens=None, route_tokens=None,
            weights_key: str | None = None, check_perm: bool = True, label: str = ""):
    """Compare GPU results with the oracle.

    Routing on rows `route_tokens` (all rows if None), see check_routing.
    Layer outputs on rows `tokens` (all if None):
      graded:  max |out_gpu - out_oracle| <= tol * RMS(y_oracle) against the
               exact (fp64) oracle, tol = 1e-5 (fp32), 2e-2 (bf16), 5e-2
               (MXFP4, on the same dequantised bits);
      reported: the same against the oracle's bf16-dataflow mode.
    Tokens whose GPU experts differ from the oracle's (only near-ties can)
    are evaluated by the oracle with the GPU's experts.  Permutation:
    bit-exact against the oracle's permutation of the GPU's own indices.
    weights_key: which stored form of the big weights the GPU ran, e.g. "mxfp4".
    """
    T = x.shape[0]
    tok = np.arange(T, dtype=np.int64) if tokens is None else np.asarray(tokens, np.int64)
    rtok = np.arange(T, dtype=np.int64) if route_tokens is None else np.asarray(route_tokens, np.int64)
    t = dict(host)
    if weights_key:
        for k_ in ("down_w", "w1", "w2", "up_w"):
            if k_ + "@" + weights_key in host:
                t[k_] = host[k_ + "@" + weights_key]
    u_orc = None
    if p.in_norm != "none" and p.act == "bf16" and "u" in gpu:
        u_orc = oracle.branch_input(oracle_cfg(p), dict(t, x=x))  # every row, once
    excluded, r_logits, same_u = check_routing(p, t, x, gpu, rtok, label, u_orc)
    if "logits" in gpu and "u" in gpu:
        known = None
        if len(rtok) == T and (rtok == np.arange(T)).all():  # the oracle's logits of every token, from its u
            if p.in_norm == "none":
                known = (r_logits, (gpu["u"] == x).all(axis=1))
            elif p.act == "bf16":
                known = (r_logits, same_u)
        check_router_stage(p, t, gpu, label, known)
        check_input_norm(p, t, x, gpu, label, u_orc)
    t["x"] = x
    cfg = oracle_cfg(p)
    gidx = gpu["topk_idx"][tok]
    refs = {}
    ndf = min(len(tok), DATAFLOW_TOKENS)  # the diagnostic dataflow mode runs on a prefix of the sample
    q8 = p.act_quant == "mxfp8" and "zq" in gpu
    if q8:
        # the device's quantized expert inputs of the compared tokens: z, and the hidden activation of every
        # selected expert in slot order (row pos[t, j] of the permuted buffer)
        zq_dev = oracle.decode_matrix(gpu["zq"], "mxfp8", T, p.L)[tok]
        TK, F_ = T * p.k, p.F
        prow = gpu["pos"][tok].reshape(-1)
        abuf = np.concatenate([gpu["actq"][:TK * F_].reshape(TK, F_)[prow].reshape(-1),
                               gpu["actq"][TK * F_:].reshape(TK, F_ // 32)[prow].reshape(-1)])
        aq_dev = oracle.decode_matrix(abuf, "mxfp8", len(prow), F_).reshape(len(tok), p.k, F_)
    nzf = 0
    for mode, mirror, tt in (("exact", False, tok), ("dataflow", True, tok[:ndf])):
        r = oracle.forward(cfg, t, tokens=tt, mirror=mirror, want_z=q8, want_a=q8)
        y_ref, out_ref, ypre = r["y"].copy(), r["out"].copy(), r["ypre"].copy()
        nt = len(tt)
        diff = ~(gidx[:nt] == r["idx"]).all(axis=1)
        qdiff = np.zeros(nt, bool)
        if q8:
            # A token whose quantized expert inputs differ from the oracle's is evaluated on the device's, as
            # a near-tie token is on the device's experts: an E4M3 code (or a block's shared scale) decided on
            # either side of a rounding point by a one-ulp difference of the stored value, from fp32 against
            # fp64 sums, from a flip of u, or within the scaled MFMA's own error bound.
            qdiff = ~(zq_dev[:nt] == r["z"]).all(axis=1) | ~(aq_dev[:nt] == r["a"]).all(axis=(1, 2))
        redo = np.flatnonzero(diff | qdiff)
        if mode == "exact" and q8:
            unforced = np.abs(gpu["out"][tt] - r["out"]).max() / np.sqrt(np.mean(r["y"] ** 2))
        if redo.size:
            rf = oracle.forward(cfg, t, tokens=tt[redo], forced=gidx[redo], mirror=mirror,
                                forced_z=zq_dev[redo] if q8 else None, forced_a=aq_dev[redo] if q8 else None)
            y_ref[redo], out_ref[redo], ypre[redo] = rf["y"], rf["out"], rf["ypre"]
        if mode == "exact":
            nzf = int(qdiff.sum())
        refs[mode] = (y_ref, out_ref, int(diff.sum()), ypre)
    y_ex, out_ex, nforced, ypre = refs["exact"]
    y_df, out_df, _, ypre_df = refs["dataflow"]
    rms = float(np.sqrt(np.mean(y_ex ** 2)))
    kind = p.weights if p.act == "bf16" else "f32"
    tol, tol_df = TOL[kind], TOL_DATAFLOW[kind]
    allow_y, allow_out = output_norm_allowance(p, t, ypre)
    dout, dy = np.abs(gpu["out"][tok] - out_ex), np.abs(gpu["y"][tok] - y_ex)
    e_out = float(np.maximum(dout - allow_out, 0).max()) / rms
    e_y = float(np.maximum(dy - allow_y, 0).max()) / rms
    allow_y_df, allow_out_df = output_norm_allowance(p, t, ypre_df)
    e_out_df = float(np.maximum(np.abs(gpu["out"][tok[:ndf]] - out_df) - allow_out_df, 0).max()) / rms
    e_y_df = float(np.maximum(np.abs(gpu["y"][tok[:ndf]] - y_df) - allow_y_df, 0).max()) / rms
    beyond = float((dout > tol * rms).mean())
    if q8:
        say("%s: %d of %d tokens evaluated on the device's quantized expert inputs (an MXFP8 code differs); "
            "without that, max|dout|/rms = %.3g (reported)" % (label, nzf, len(tok), unforced))
    say("%s: routed=%d (excluded %d) compared=%d forced=%d rms(y)=%.4g | exact: max|dout|/rms=%.3g (tol %.0e) "
        "max|dy|/rms=%.3g | bf16-dataflow: max|dout|/rms=%.3g max|dy|/rms=%.3g (tol %.0e)%s" % (
            label, len(rtok), excluded, len(tok), nforced, rms, e_out, tol, e_y, e_out_df, e_y_df, tol_df,
            " | output-norm flips: raw max|dout|/rms=%.3g, beyond tol %.4f%%" % (float(dout.max()) / rms,
                                                                           100 * beyond)
            if p.out_norm != "none" else ""))
    if e_out > tol:
        worst = np.argsort(-np.maximum(dout - allow_out, 0).max(axis=1))[:5]
        for w_ in worst:
            say("  worst token %d: max|dout|/rms %.3g, experts %s" % (
                tok[w_], float(np.maximum(dout[w_] - allow_out if np.ndim(allow_out) < 2 else dout[w_] - allow_out[w_],
                                          0).max()) / rms, gidx[w_].tolist()))
    assert e_out <= tol, "%s out error %.3g * RMS(y) > %.0e" % (label, e_out, tol)
    assert beyond <= FLIP_OUT_FRACTION, "%s: %.3g of the outputs beyond the tolerance" % (label, beyond)
    if kind == "f32":
        assert e_y <= tol, "%s y error %.3g * RMS(y) > %.0e" % (label, e_y, tol)
    if check_perm:
        pr = oracle.permute(gpu["topk_idx"], p.n)
        np.testing.assert_array_equal(gpu["expert_counts"], pr["counts"], err_msg=label + " counts")
        np.testing.assert_array_equal(gpu["expert_offsets"], pr["offsets"], err_msg=label + " offsets")
        np.testing.assert_array_equal(gpu["perm_tok"], pr["perm_tok"], err_msg=label + " perm_tok")
        np.testing.assert_array_equal(gpu["perm_slot"], pr["perm_slot"], err_msg=label + " perm_slot")
    return {"err_out": e_out, "err_y": e_y, "err_out_df": e_out_df, "err_y_df": e_y_df, "excluded": excluded}


# ---------------------------------------------------------------------------
# Stage checks: each device stage against the exact function of the device's
# own stage input, rounded where the device stores the result.  Agreement is
# to one bf16 ulp on a small fraction of elements: an fp32 (device) and an
# fp64 sum of the same products can straddle a bf16 rounding boundary.
# ---------------------------------------------------------------------------

FLIP_FRACTION = 5e-3


def bf16f(a: np.ndarray) -> np.ndarray:
    return synthetic.bf16_to_f32(np.ascontiguousarray(a).view(np.uint16)).astype(np.float64)


def round_bf16(v: np.ndarray) -> np.ndarray:
    """bf16 RNE of float64 values (torch's conversion, a library routine)."""
    return torch.from_numpy(np.asarray(v, np.float64)).to(torch.bfloat16).to(torch.float64).numpy()


def round_f16(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(v, np.float64)).to(torch.float16).to(torch.float64).numpy()


def f16f(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint16).view(np.float16).astype(np.float64)


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def ulp_f16(v: np.ndarray) -> np.ndarray:
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -14)))
    return 2.0 ** (e - 10)


def interm_ops(p):
    """(decode, round, ulp) of the dtype the device keeps z, act and m in."""
    if p.interm == "bf16":
        return bf16f, round_bf16, ulp_bf16
    return f16f, round_f16, ulp_f16


def weight_rows(host: dict, key: str, fmt: str, rows_total: int, K: int, row0: int, nrows: int) -> np.ndarray:
    """Rows [row0, row0+nrows) of a stored [rows_total][K] weight, as float64."""
    w = host[key]
    if fmt == "mxfp4":
        codes = w[:rows_total * K // 2].reshape(rows_total, K // 2)[row0:row0 + nrows]
        sc = w[rows_total * K // 2:].reshape(rows_total, K // 32)[row0:row0 + nrows]
        buf = np.concatenate([codes.reshape(-1), sc.reshape(-1)])
        return oracle.decode_matrix(buf, "mxfp4", nrows, K)
    flat = w.reshape(-1, K)[row0:row0 + nrows]
    return bf16f(flat) if flat.dtype == np.uint16 else flat.astype(np.float64)


# The scaled fp8 x fp4 MFMA (MXFP8 activations on the large tiles) does not
# sum its products in full fp32: a one-wave probe of the instruction on
# random E4M3/E2M1 operands and scales put its error at up to 2^-11.6 of the
# largest product of the 64-deep instruction and 2.4e-4 of the sum of the
# products' magnitudes.  Its GEMM outputs are therefore allowed, on top of
# the rounding of the stored value, 2^-11 times the sum of |a_k b_k| over K.
MX8_MFMA_REL = 2.0 ** -11


def _flips(name, got, ref, label, ulp=ulp_bf16, floor=None, extra=None):
    """got vs ref: equal except one-ulp flips; `floor` (per row) admits the
    absolute error of an fp32 sum where the result nearly cancels; `extra`
    (per element) an error bound of the arithmetic that produced got."""
    d = np.abs(got - ref)
    lim = 1.01 * ulp(ref)
    if floor is not None:
        lim = np.maximum(lim, floor[:, None])
    if extra is not None:
        lim = lim + extra
    bad = d > lim
    frac = float((d > 0).mean())
    say("  stage %-4s %s: differing %.4f%%, beyond 1 ulp %d" % (name, label, 100 * frac, int(bad.sum())))
    for r_, c_ in list(zip(*np.nonzero(bad)))[:6]:
        say("    row %d col %d: device %.9g reference %.9g |d| %.3g limit %.3g" % (
            r_, c_, got[r_, c_], ref[r_, c_], d[r_, c_], lim[r_, c_]))
    assert not bad.any(), "%s stage %s: %d elements beyond one bf16 ulp" % (label, name, int(bad.sum()))
    if extra is None:  # with an arithmetic error bound, the element-wise bound is the check
        assert frac <= FLIP_FRACTION, "%s stage %s: %.3g of elements differ" % (label, name, frac)


def check_stages(p: synthetic.Preset, host: dict, x: np.ndarray, gpu: dict, tokens, label: str = ""):
    """Stage checks on tokens `tokens` and their (token, slot) rows."""
    tok = np.asarray(tokens, np.int64)
    fmt = p.weights
    dec, rnd, ulp = interm_ops(p)
    rowfloor = lambda a: 3e-5 * np.sqrt(np.mean(a ** 2, axis=1))
    d, L, F, n, k = p.d, p.L, p.F, p.n, p.k
    xf = bf16f(x[tok])
    # the down-projection of the device's own u (the input norm is checked on its own), or of the
    # exact input norm (fp64) when the device's u was not captured
    if "u" in gpu:
        u = bf16f(gpu["u"][tok])
    elif p.in_norm != "none":
        gam = 1.0 + host["gamma_in"].astype(np.float64)
        if p.in_norm == "centered":
            u = gam * xf / np.sqrt((xf * xf).mean(1, keepdims=True) + p.eps_in)
        else:
            s_ = round_bf16(gam * xf)
            u = s_ / np.sqrt((s_ * s_).mean(1, keepdims=True) + p.eps_in)
        u = round_bf16(u)
    else:
        u = xf
    Wd = weight_rows(host, "down_w", fmt, L, d, 0, L)
    zexact = u @ Wd.T
    if p.latent_norm == "centered":
        # the device stores P_down u in the intermediate type, then normalises it
        zr = rnd(zexact)
        zexact = (1.0 + host["gamma_lat"].astype(np.float64)) * zr / np.sqrt((zr * zr).mean(1, keepdims=True)
                                                                            + p.eps_latent)
    zref = rnd(zexact)
    zg = dec(gpu["z"][tok])
    if ("u" not in gpu and p.in_norm != "none") or p.latent_norm != "none":
        # an exact u may differ from the device's by one bf16 ulp in a few elements: z within 1e-3
        # relative of the row; the latent pre-norm rounds twice (P_down u, then its normalised value):
        # one more ulp of z
        dz = np.abs(zg - zexact)
        nulp = 2 if p.latent_norm != "none" else 1
        rel = 1e-3 if ("u" not in gpu and p.in_norm != "none") else 3e-5
        lim = rel * np.sqrt(np.mean(zexact ** 2, axis=1))[:, None] + nulp * ulp(zexact)
        say("  stage z    %s: max |dz| / limit %.3f" % (label, float((dz / lim).max())))
        assert (dz <= lim).all(), label + " stage z"
    else:
        _flips("z", zg, zref, label, ulp, rowfloor(zexact))
    del Wd
    pos = gpu["pos"][tok]
    rows = pos.reshape(-1)
    offs = gpu["expert_offsets"]
    eid = np.searchsorted(offs, rows, side="right") - 1
    zfull = dec(gpu["z"])
    ptok = gpu["perm_tok"]
    actg = dec(gpu["act"][rows])
    Sg = bf16f(gpu["S"][rows])
    act_in = actg  # what GEMM2 multiplies
    if p.act_quant == "mxfp8":
        # the quantized z and SwiGLU output: bit for bit the oracle's quantizer applied to the device's own
        # stored values (the same inputs: a decision taken in the same precision on both sides)
        T = gpu["z"].shape[0]
        TK = gpu["act"].shape[0]
        zq = oracle.decode_matrix(gpu["zq"], "mxfp8", T, L)
        zq_ref, zX = oracle.mxfp8_quantize(zfull)
        np.testing.assert_array_equal(zq, zq_ref, err_msg=label + " stage zq (values)")
        np.testing.assert_array_equal(gpu["zq"][T * L:].reshape(T, L // 32).astype(np.int32),
                                      np.maximum(zX + 127, 0), err_msg=label + " stage zq (scales)")
        ascales = gpu["actq"][TK * F:].reshape(TK, F // 32).astype(np.int32)
        acodes = gpu["actq"][:TK * F].reshape(TK, F)
        # every row up to 16384 rows; beyond, a seeded sample of 16384 rows and the checked tokens' rows
        arows = np.arange(TK) if TK <= 16384 else np.unique(np.concatenate([
            np.random.default_rng(3).choice(TK, 16384, replace=False), rows]))
        for a in range(0, len(arows), 8192):
            r_ = arows[a:a + 8192]
            buf = np.concatenate([acodes[r_].reshape(-1), gpu["actq"][TK * F:].reshape(TK, F // 32)[r_].reshape(-1)])
            got = oracle.decode_matrix(buf, "mxfp8", len(r_), F)
            ref, aX = oracle.mxfp8_quantize(dec(gpu["act"][r_]))
            np.testing.assert_array_equal(got, ref, err_msg=label + " stage actq (values)")
            np.testing.assert_array_equal(ascales[r_], np.maximum(aX + 127, 0), err_msg=label + " stage actq (scales)")
        say("  stage zq/actq %s: MXFP8 codes and scales of %d + %d rows bit-exact" % (label, T, len(arows)))
        zfull = zq
        abuf = np.concatenate([gpu["actq"][:TK * F].reshape(TK, F)[rows].reshape(-1),
                               gpu["actq"][TK * F:].reshape(TK, F // 32)[rows].reshape(-1)])
        act_in = oracle.decode_matrix(abuf, "mxfp8", len(rows), F)
    act_ref = np.zeros_like(actg)
    o_ref = np.zeros_like(Sg)
    q8 = p.act_quant == "mxfp8"
    act_err = np.zeros_like(actg) if q8 else None  # the scaled MFMA's bound, carried through SwiGLU
    o_err = np.zeros_like(Sg) if q8 else None
    for e in np.unique(eid):
        sel = np.flatnonzero(eid == e)
        W1 = weight_rows(host, "w1", fmt, n * 2 * F, L, e * 2 * F, 2 * F)
        zin = zfull[ptok[rows[sel]]]
        g_, v_ = zin @ W1[:F].T, zin @ W1[F:].T
        sg = 1 / (1 + np.exp(-g_))
        act_ref[sel] = g_ * sg * v_
        W2 = weight_rows(host, "w2", fmt, n * L, F, e * L, L)
        o_ref[sel] = act_in[sel] @ W2.T
        if q8:
            dg = MX8_MFMA_REL * (np.abs(zin) @ np.abs(W1[:F]).T)
            dv = MX8_MFMA_REL * (np.abs(zin) @ np.abs(W1[F:]).T)
            dsilu = sg * (1 + g_ * (1 - sg))  # d silu / dg
            act_err[sel] = np.abs(dsilu * v_) * dg + np.abs(g_ * sg) * dv + dg * dv
            o_err[sel] = MX8_MFMA_REL * (np.abs(act_in[sel]) @ np.abs(W2).T)
    _flips("act", actg, rnd(act_ref), label, ulp, rowfloor(act_ref), act_err)
    gam = 1.0 + (host["gamma_ex"].astype(np.float64) if "gamma_ex" in host else 0.0)
    S_ref = round_bf16(gam * o_ref)
    _flips("S", Sg, S_ref, label, ulp_bf16, rowfloor(gam * o_ref), None if o_err is None else np.abs(gam) * o_err)
    if p.expert_norm != "none":
        sq = (Sg if p.expert_norm == "input_scaled" else o_ref) ** 2
        ssq_ref = sq.reshape(len(rows), L // 16, 16).sum(2)
        np.testing.assert_allclose(gpu["ssq"][rows], ssq_ref, rtol=2e-5, atol=1e-30, err_msg=label + " ssq")
        r = 1.0 / np.sqrt(gpu["ssq"][rows].astype(np.float64).sum(1) / L + p.eps_expert)
    else:
        r = np.ones(len(rows))
    coef = (gpu["topk_w"][tok].reshape(-1).astype(np.float64) * r).reshape(len(tok), k)
    m_exact = np.einsum("tj,tjl->tl", coef, Sg.reshape(len(tok), k, L))
    mg = dec(gpu["m"][tok])
    _flips("m", mg, rnd(m_exact), label, ulp, rowfloor(m_exact))
    Wu = weight_rows(host, "up_w", fmt, d, L, 0, d)
    y_ref = mg @ Wu.T
    yg = gpu["y"][tok].astype(np.float64)
    if p.out_norm != "none":
        # the epilogue stores s = bf16((1 + gamma) y); b = s / rms (of s, or of y for the centered form)
        gam = 1.0 + host["gamma_out"].astype(np.float64)
        s_ref = round_bf16(gam * y_ref)
        base = s_ref if p.out_norm == "input_scaled" else y_ref
        inv = 1.0 / np.sqrt((base * base).mean(1, keepdims=True) + p.eps_out)
        b_ref = s_ref * inv
        rms = float(np.sqrt(np.mean(b_ref ** 2)))
        # s may sit one bf16 ulp away where y straddles a rounding boundary
        lim = 1.01 * ulp_bf16(s_ref) * inv + 1e-5 * rms
        db = np.abs(yg - b_ref)
        flips = float((db > 0.5 * ulp_bf16(s_ref) * inv).mean())   # s one ulp apart (not a shift of inv)
        say("  stage outnorm %s: one-ulp flips of s %.4f%%, max |db| / limit %.3f" % (
            label, 100 * flips, float((db / lim).max())))
        assert (db <= lim).all(), label + " stage output norm"
        assert flips <= FLIP_FRACTION, label + " stage output norm flips"
    else:
        rms = float(np.sqrt(np.mean(y_ref ** 2)))
        assert np.abs(yg - y_ref).max() <= 1e-5 * rms, label + " stage up (y)"
    # residual gate on the device's own branch output
    if p.res_gate == "linear":
        out_ref = xf + host["gate"].astype(np.float64) * yg
    elif p.res_gate == "muse":
        w = host["gate"].astype(np.float64) / p.res_tau
        beta = 1.0 / (1.0 + np.exp(-w))
        alpha = np.sqrt(np.maximum(1.0 / (1.0 + np.exp(w)) * (1.0 + beta), p.res_floor))
        out_ref = alpha * xf + beta * yg
    else:
        out_ref = yg
    assert np.abs(gpu["out"][tok] - out_ref).max() <= 1e-5 * max(rms, 1.0), label + " stage residual gate (out)"
