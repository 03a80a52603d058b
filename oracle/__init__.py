"""CPU oracle for the latent sparse mixture-of-experts layer (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package; the product path
(``sparse_mixture_experts_router_amd``) never does.  The arithmetic lives in
``moe_oracle.c`` (fp64, plain loops, each function citing the page it
follows); this file only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

F32, BF16, MXFP4, F16, MXFP8 = 0, 1, 2, 3, 4
NORM_NONE, NORM_CENTERED, NORM_INPUT_SCALED = 0, 1, 2
RELU, SWIGLU = 0, 1
RES_NONE, RES_LINEAR, RES_MUSE = 0, 1, 2
ROUTER_SOFTMAX, ROUTER_SIGMOID = 0, 1

_DT = {"f32": F32, "bf16": BF16, "mxfp4": MXFP4, "f16": F16, "mxfp8": MXFP8}
_NORM = {"none": NORM_NONE, "centered": NORM_CENTERED, "input_scaled": NORM_INPUT_SCALED}
_KIND = {"relu2": RELU, "swiglu3": SWIGLU}
_RES = {"none": RES_NONE, "linear": RES_LINEAR, "muse": RES_MUSE}
_ROUTER = {"softmax": ROUTER_SOFTMAX, "sigmoid": ROUTER_SIGMOID}
_AQ = {"none": 0, "mxfp8": 1}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (fp64 C + OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-Wno-unknown-pragmas", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Desc(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int64), ("L", ctypes.c_int64), ("n", ctypes.c_int64),
                ("k", ctypes.c_int64), ("F", ctypes.c_int64),
                ("kind", ctypes.c_int32), ("act", ctypes.c_int32), ("wdt", ctypes.c_int32),
                ("rdt", ctypes.c_int32), ("in_norm", ctypes.c_int32), ("ex_norm", ctypes.c_int32),
                ("res_gate", ctypes.c_int32), ("bias_in_weights", ctypes.c_int32),
                ("eps_in", ctypes.c_double), ("eps_ex", ctypes.c_double),
                ("mirror", ctypes.c_int32), ("interm", ctypes.c_int32),
                ("router_fn", ctypes.c_int32), ("out_mult", ctypes.c_double), ("rsf", ctypes.c_double),
                ("lat_norm", ctypes.c_int32), ("out_norm", ctypes.c_int32),
                ("eps_lat", ctypes.c_double), ("eps_out", ctypes.c_double),
                ("tau", ctypes.c_double), ("floor_", ctypes.c_double), ("act_quant", ctypes.c_int32)]


class _Tensors(ctypes.Structure):
    _fields_ = [(nm, ctypes.c_void_p) for nm in
                ("x", "router_w", "down_w", "w1", "w2", "up_w", "bias", "gamma_in", "gamma_ex", "gate",
                 "gamma_lat", "gamma_out")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("MOE_ORACLE_LIB")  # a separately built copy (e.g. a sanitizer build)
        if not path:
            path = build()  # compiles only when the library is missing or older than its source
        _lib = ctypes.CDLL(path)
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        _lib.orc_forward.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Tensors), vp, i64, vp, i32,
                                     vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        _lib.orc_permute.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp]
        _lib.orc_rms_centered.argtypes = [vp, vp, i64, dbl, vp]
        _lib.orc_rms_input_scaled.argtypes = [vp, vp, i64, dbl, ctypes.c_int, vp]
        _lib.orc_topk.argtypes = [vp, i64, i64, vp, vp]
        _lib.orc_softmax_kept.argtypes = [vp, vp, i64, vp]
        _lib.orc_gate_dense.argtypes = [vp, i64, i64, vp]
        _lib.orc_decode_matrix.argtypes = [vp, i32, i64, i64, vp]
        _lib.orc_round_bf16.argtypes = [dbl]
        _lib.orc_round_bf16.restype = dbl
        _lib.orc_round_f16.argtypes = [dbl]
        _lib.orc_round_f16.restype = dbl
        _lib.orc_router_scores.argtypes = [ctypes.POINTER(_Desc), vp, vp, vp, vp]
        _lib.orc_router_weights.argtypes = [ctypes.POINTER(_Desc), vp, vp, i64, vp]
        _lib.orc_muse_gate_coeffs.argtypes = [dbl, dbl, dbl, vp, vp]
        _lib.orc_threads.restype = ctypes.c_int
        _lib.orc_branch_input.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Tensors), vp, i64, vp]
        _lib.orc_mxfp8_quantize.argtypes = [vp, i64, vp]
    return _lib


def threads() -> int:
    """Threads the oracle's parallel loops run on."""
    return int(lib().orc_threads())


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def make_desc(cfg: dict, mirror: bool = False) -> _Desc:
    """cfg keys: d, L, n, k, F, kind, act, weights, router_w, in_norm,
    expert_norm, res_gate, eps_in, eps_expert, bias_in_weights; optional
    router_fn ("softmax"), out_mult (1), routed_scale (1), latent_norm
    ("none"), out_norm ("none"), eps_latent, eps_out (1e-5), res_tau (0.3),
    res_floor (1e-3), act_quant ("none" | "mxfp8": the expert GEMMs read
    MXFP8 activations)."""
    return _Desc(d=cfg["d"], L=cfg["L"], n=cfg["n"], k=cfg["k"], F=cfg["F"],
                 kind=_KIND[cfg["kind"]], act=_DT[cfg["act"]], wdt=_DT[cfg["weights"]],
                 rdt=_DT[cfg["router_w"]], in_norm=_NORM[cfg["in_norm"]],
                 ex_norm=_NORM[cfg["expert_norm"]], res_gate=_RES[cfg["res_gate"]],
                 bias_in_weights=int(cfg.get("bias_in_weights", 0)),
                 eps_in=float(cfg["eps_in"]), eps_ex=float(cfg["eps_expert"]),
                 mirror=int(mirror), interm=_DT[cfg.get("interm", "bf16")] if cfg["act"] == "bf16" else F32,
                 router_fn=_ROUTER[cfg.get("router_fn", "softmax")], out_mult=float(cfg.get("out_mult", 1.0)),
                 rsf=float(cfg.get("routed_scale", 1.0)), lat_norm=_NORM[cfg.get("latent_norm", "none")],
                 out_norm=_NORM[cfg.get("out_norm", "none")], eps_lat=float(cfg.get("eps_latent", 1e-5)),
                 eps_out=float(cfg.get("eps_out", 1e-5)), tau=float(cfg.get("res_tau", 0.3)),
                 floor_=float(cfg.get("res_floor", 1e-3)), act_quant=_AQ[cfg.get("act_quant", "none")])


_KEEP = []


def forward(cfg: dict, t: dict, tokens=None, forced=None, dense: bool = False, mirror: bool = False,
            want_outputs: bool = True, want_z: bool = False, forced_z=None, want_a: bool = False,
            forced_a=None) -> dict:
    """Run the oracle on host arrays.

    t: dict with numpy arrays (raw stored forms: uint16 bf16 bits, float32,
    or uint8 MXFP4 buffers) under keys x, router_w, down_w, w1, w2, up_w and
    optional float32 bias, gamma_in, gamma_ex, gate, gamma_lat, gamma_out.
    tokens: int64 array of token ids (None: all T rows of x).
    forced: int32 [ntok][k] expert ids (None: route).
    forced_z: float64 [ntok][Dx] expert-space inputs to use (None: compute).
    want_z: also return z, the expert-space input the experts read.
    forced_a: float64 [ntok][k][F] hidden activations of the selected experts
    to use (None: compute); want_a: also return a, the ones the experts read.
    Outputs: logits, idx, w, margin; with want_outputs also y (the branch
    output entering the residual gate), out, and ypre (the branch output
    before the output norm).
    """
    desc = make_desc(cfg, mirror)
    T = t["x"].shape[0]
    tok = np.arange(T, dtype=np.int64) if tokens is None else _c(tokens, np.int64)
    ntok = tok.shape[0]
    arrs = {}
    for nm in ("x", "router_w", "down_w", "w1", "w2", "up_w"):
        a = t.get(nm)
        arrs[nm] = None if a is None else np.ascontiguousarray(a)
    for nm in ("bias", "gamma_in", "gamma_ex", "gate", "gamma_lat", "gamma_out"):
        a = t.get(nm)
        arrs[nm] = None if a is None else _c(a, np.float32)
    tens = _Tensors(**{nm: _p(a) for nm, a in arrs.items()})
    d, n, k = cfg["d"], cfg["n"], cfg["k"]
    res = {
        "logits": np.zeros((ntok, n), np.float32),
        "idx": np.zeros((ntok, k), np.int32),
        "w": np.zeros((ntok, k), np.float64),
        "margin": np.zeros((ntok,), np.float64),
    }
    if want_outputs:
        res["y"] = np.zeros((ntok, d), np.float64)
        res["out"] = np.zeros((ntok, d), np.float64)
        res["ypre"] = np.zeros((ntok, d), np.float64)
    fz = None if forced is None else _c(forced, np.int32)
    Dx = cfg["L"] if cfg["L"] else cfg["d"]
    if want_z:
        res["z"] = np.zeros((ntok, Dx), np.float64)
    fzz = None if forced_z is None else _c(forced_z, np.float64)
    if want_a:
        res["a"] = np.zeros((ntok, k, cfg["F"]), np.float64)
    faa = None if forced_a is None else _c(forced_a, np.float64)
    rc = lib().orc_forward(ctypes.byref(desc), ctypes.byref(tens), _p(tok), ntok, _p(fz), int(dense),
                           _p(res.get("y")), _p(res.get("out")), _p(res["logits"]), _p(res["idx"]),
                           _p(res["w"]), _p(res["margin"]), _p(res.get("ypre")), _p(res.get("z")), _p(fzz),
                           _p(res.get("a")), _p(faa))
    assert rc == 0
    res["tokens"] = tok
    return res


def branch_input(cfg: dict, t: dict, tokens=None) -> np.ndarray:
    """The branch input u of rows `tokens` (all rows if None): x, or its
    input norm rounded to the input dtype, as float64 [ntok][d]."""
    desc = make_desc(cfg)
    x = np.ascontiguousarray(t["x"])
    tok = np.arange(x.shape[0], dtype=np.int64) if tokens is None else _c(tokens, np.int64)
    g = None if t.get("gamma_in") is None else _c(t["gamma_in"], np.float32)
    tens = _Tensors(x=_p(x), gamma_in=_p(g))
    out = np.zeros((tok.shape[0], cfg["d"]), np.float64)
    lib().orc_branch_input(ctypes.byref(desc), ctypes.byref(tens), _p(tok), tok.shape[0], _p(out))
    return out


def mxfp8_quantize(v):
    """MXFP8 (E4M3 elements, one power-of-two scale per 32 consecutive
    values of the last axis): (dequantized values, scale exponents X)."""
    v = np.array(v, np.float64, copy=True)
    shape = v.shape
    assert shape[-1] % 32 == 0
    flat = np.ascontiguousarray(v.reshape(-1))
    X = np.zeros(flat.size // 32, np.int32)
    lib().orc_mxfp8_quantize(_p(flat), flat.size, _p(X))
    return flat.reshape(shape), X.reshape(shape[:-1] + (shape[-1] // 32,))


def router_scores(cfg: dict, logits, bias=None):
    """Selection scores and weight basis (float64 [rows][n] each) of fp32
    logits [rows][n] under the cfg's router function."""
    desc = make_desc(cfg)
    lg = np.atleast_2d(_c(logits, np.float32))
    b = None if bias is None else _c(bias, np.float32)
    sel = np.zeros(lg.shape, np.float64)
    H = np.zeros(lg.shape, np.float64)
    for r in range(lg.shape[0]):
        lr, sr, hr = lg[r], sel[r], H[r]
        lib().orc_router_scores(ctypes.byref(desc), _p(lr), _p(b), _p(sr), _p(hr))
    return sel, H


def router_weights(cfg: dict, H, idx) -> np.ndarray:
    """Weights of the kept experts idx [k] from the weight basis H [n]."""
    desc = make_desc(cfg)
    H = _c(H, np.float64)
    idx = _c(idx, np.int32)
    w = np.zeros(idx.shape[0], np.float64)
    lib().orc_router_weights(ctypes.byref(desc), _p(H), _p(idx), idx.shape[0], _p(w))
    return w


def muse_gate_coeffs(g, tau: float = 0.3, floor: float = 1e-3):
    """(alpha, beta) of the residual gate for each value of g."""
    g = np.atleast_1d(np.asarray(g, np.float64))
    al = np.zeros_like(g)
    be = np.zeros_like(g)
    a_, b_ = ctypes.c_double(), ctypes.c_double()
    for i, gv in enumerate(g):
        lib().orc_muse_gate_coeffs(float(gv), tau, floor, ctypes.byref(a_), ctypes.byref(b_))
        al[i], be[i] = a_.value, b_.value
    return al, be


def permute(idx: np.ndarray, n: int) -> dict:
    idx = _c(idx, np.int32)
    T, k = idx.shape
    out = {"counts": np.zeros(n, np.int32), "offsets": np.zeros(n + 1, np.int32),
           "perm_tok": np.zeros(T * k, np.int32), "perm_slot": np.zeros(T * k, np.int32),
           "pos": np.zeros((T, k), np.int32)}
    rc = lib().orc_permute(_p(idx), T, k, n, _p(out["counts"]), _p(out["offsets"]), _p(out["perm_tok"]),
                           _p(out["perm_slot"]), _p(out["pos"]))
    if rc != 0:
        raise ValueError("expert id out of range")
    return out


def rms_centered(x, gamma, eps: float = 0.0) -> np.ndarray:
    x = _c(x, np.float64)
    g = None if gamma is None else _c(gamma, np.float32)
    out = np.zeros_like(x)
    lib().orc_rms_centered(_p(x), _p(g), x.shape[0], eps, _p(out))
    return out


def rms_input_scaled(x, gamma, eps: float = 0.0, act: str | None = None) -> np.ndarray:
    x = _c(x, np.float64)
    g = None if gamma is None else _c(gamma, np.float32)
    out = np.zeros_like(x)
    lib().orc_rms_input_scaled(_p(x), _p(g), x.shape[0], eps, -1 if act is None else _DT[act], _p(out))
    return out


def topk(score, k: int):
    s = _c(score, np.float64)
    idx = np.zeros(k, np.int32)
    margin = np.zeros(1, np.float64)
    lib().orc_topk(_p(s), s.shape[0], k, _p(idx), _p(margin))
    return idx, float(margin[0])


def softmax_kept(H, idx) -> np.ndarray:
    H = _c(H, np.float64)
    idx = _c(idx, np.int32)
    w = np.zeros(idx.shape[0], np.float64)
    lib().orc_softmax_kept(_p(H), _p(idx), idx.shape[0], _p(w))
    return w


def gate_dense(H, k: int) -> np.ndarray:
    H = _c(H, np.float64)
    G = np.zeros_like(H)
    lib().orc_gate_dense(_p(H), H.shape[0], k, _p(G))
    return G


def decode_matrix(buf: np.ndarray, dt: str, rows: int, K: int) -> np.ndarray:
    buf = np.ascontiguousarray(buf)
    out = np.zeros((rows, K), np.float64)
    lib().orc_decode_matrix(_p(buf), _DT[dt], rows, K, _p(out))
    return out


def round_bf16(v: float) -> float:
    return lib().orc_round_bf16(float(v))


def round_f16(v: float) -> float:
    return lib().orc_round_f16(float(v))
