"""Helpers of the GPU parity tests: move seeded host inputs to the device,
run the HIP layer through the C ABI, and compare with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import sparse_mixture_experts_router_amd as moe
import synthetic

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
    return moe.make_desc(p.chunk_T if T is None else T, p.d, p.L, p.n, p.k, p.F, expert_kind=p.kind, act=p.act,
                         router=p.router_w, weights=p.weights, in_norm=p.in_norm, expert_norm=p.expert_norm,
                         res_gate=p.res_gate, bias_in_weights=p.bias_in_weights, eps_in=p.eps_in,
                         eps_expert=p.eps_expert)


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
                "gamma_expert": self.dev.get("gamma_ex"), "res_gate": self.dev.get("gate")}


def run(layer: DeviceLayer, x: np.ndarray, dbg: bool = True, workspace=None):
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
             "y": torch.empty((T, p.d), dtype=torch.float32, device="cuda")}
    dv = layer.dev
    moe.moe_layer_forward(desc, xd, dv["router_w"], dv.get("down_w"), dv["w1"], dv["w2"], dv.get("up_w"),
                          layer.gains(), out, workspace=workspace, dbg=D)
    torch.cuda.synchronize()
    res = {"out": out.cpu().numpy()}
    if dbg:
        for k_, v in D.items():
            res[k_] = v.cpu().numpy()
    return res


def oracle_cfg(p: synthetic.Preset) -> dict:
    return p.cfg()


def check_routing(p, host, x, gpu, tokens, label=""):
    """Routing of rows `tokens`: expert sets bit-exact where the oracle's
    k-th/(k+1)-th score margin is >= 1e-4, order bit-exact where every
    adjacent gap of the top k+1 scores is >= 1e-4; gate weights to 2e-5."""
    t = dict(host)
    t["x"] = x
    r = oracle.forward(oracle_cfg(p), t, tokens=tokens, want_outputs=False)
    gidx = gpu["topk_idx"][tokens]
    s = r["logits"].astype(np.float32)
    if "bias" in host:
        s = (s + host["bias"].astype(np.float32)).astype(np.float32)
    clean = r["margin"] >= MARGIN_EXCLUDE
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
    same = (gidx == r["idx"]).all(axis=1)
    np.testing.assert_allclose(gpu["topk_w"][tokens][same], r["w"][same], rtol=0, atol=2e-5,
                               err_msg=label + " gate weights")
    return int((~clean).sum())


def compare(p: synthetic.Preset, host: dict, x: np.ndarray, gpu: dict, tokens=None, route_tokens=None,
            weights_key: str | None = None, check_perm: bool = True, label: str = ""):
    """Compare GPU results with the oracle.

    Routing on rows `route_tokens` (all rows if None), see check_routing.
    Outputs on rows `tokens` (all if None): max |out_gpu - out_oracle| and
    max |y_gpu - y_oracle| within tol * RMS(y_oracle), where tokens whose GPU
    experts differ from the oracle's (only near-ties can) are evaluated by the
    oracle with the GPU's experts.  Permutation: bit-exact against the
    oracle's permutation of the GPU's own top-k indices.
    weights_key: which stored form of the big weights the GPU ran (the
    oracle decodes the same bits), e.g. "mxfp4".
    """
    T = x.shape[0]
    tok = np.arange(T, dtype=np.int64) if tokens is None else np.asarray(tokens, np.int64)
    rtok = np.arange(T, dtype=np.int64) if route_tokens is None else np.asarray(route_tokens, np.int64)
    t = dict(host)
    if weights_key:
        for k_ in ("down_w", "w1", "w2", "up_w"):
            if k_ + "@" + weights_key in host:
                t[k_] = host[k_ + "@" + weights_key]
    excluded = check_routing(p, t, x, gpu, rtok, label)
    t["x"] = x
    cfg = oracle_cfg(p)
    r = oracle.forward(cfg, t, tokens=tok)
    gidx = gpu["topk_idx"][tok]
    y_ref, out_ref = r["y"].copy(), r["out"].copy()
    diff = np.flatnonzero(~(gidx == r["idx"]).all(axis=1))
    if diff.size:
        rf = oracle.forward(cfg, t, tokens=tok[diff], forced=gidx[diff])
        y_ref[diff], out_ref[diff] = rf["y"], rf["out"]
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    tol = TOL[p.weights if p.act == "bf16" else "f32"]
    err_out = float(np.abs(gpu["out"][tok] - out_ref).max())
    err_y = float(np.abs(gpu["y"][tok] - y_ref).max())
    say("%s: routed=%d (excluded %d) compared=%d forced=%d rms(y)=%.4g max|dout|/rms=%.3g max|dy|/rms=%.3g "
        "(tol %.0e)" % (label, len(rtok), excluded, len(tok), diff.size, rms, err_out / rms, err_y / rms, tol))
    assert err_out <= tol * rms, "%s out error %.3g > %.3g" % (label, err_out, tol * rms)
    assert err_y <= tol * rms, "%s y error %.3g > %.3g" % (label, err_y, tol * rms)
    if check_perm:
        pr = oracle.permute(gpu["topk_idx"], p.n)
        np.testing.assert_array_equal(gpu["expert_counts"], pr["counts"], err_msg=label + " counts")
        np.testing.assert_array_equal(gpu["expert_offsets"], pr["offsets"], err_msg=label + " offsets")
        np.testing.assert_array_equal(gpu["perm_tok"], pr["perm_tok"], err_msg=label + " perm_tok")
        np.testing.assert_array_equal(gpu["perm_slot"], pr["perm_slot"], err_msg=label + " perm_slot")
    return {"err_out": err_out / rms, "err_y": err_y / rms, "excluded": excluded}
