"""Seeded synthetic inputs for the latent MoE layer (shared by tests and bench).

Holds the input recipes only: Philox4x32-10 draws keyed by (seed, tensor
name), bf16 round-to-nearest-even, the OCP MX v1.0 MXFP4 quantiser, and the
workload presets.  None of the layer's arithmetic lives here, so both the CPU
oracle and the GPU path consume exactly the same stored bits.

Workloads (the shapes and distributions of the pages' model):
  c0   tiny Shazeer layer, fp32: T=64, d=64, n=8, k=2, ReLU experts 64->128->64
  c1   816B-A42B latent layer, decode: T=64, d=8192, L=4096, F=4096, n=256, k=8
  c2   same layer, prefill: T=8192
  c3   same layer, T=16384, Zipf(1.2) selection bias 1.5*ln(rank weight)
  c4c  same layer with MXFP4 weights, 4 chunks of 8192, centered input norm
  c4i  as c4c with the input-scaled input norm
  c4q  as c4c with MXFP8 activations at the two expert GEMMs
  m1/m2  the Muse sublayer around the c1 layer at T=64 / T=8192
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=gnu11", "-Wall",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("MOE_SYNTH_LIB")  # a separately built copy (e.g. a sanitizer build)
        if not path:
            path = build()  # compiles only when the library is missing or older than its source
        _lib = ctypes.CDLL(path)
        vp, u64, i64, f32, cp = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int64, ctypes.c_float, ctypes.c_char_p
        _lib.synth_philox4x32_10.argtypes = [vp, vp, vp]
        _lib.synth_key.argtypes = [u64, cp, vp]
        _lib.synth_normal_f32.argtypes = [u64, cp, u64, u64, f32, vp]
        _lib.synth_normal_bf16.argtypes = [u64, cp, u64, u64, f32, vp]
        _lib.synth_uniform_f32.argtypes = [u64, cp, u64, u64, f32, f32, vp]
        _lib.synth_f32_to_bf16.argtypes = [vp, vp, u64]
        _lib.synth_mxfp4_quantize.argtypes = [vp, i64, i64, vp, vp]
        _lib.synth_normal_rows.argtypes = [u64, cp, i64, i64, i64, f32, vp, vp, vp]
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


# ----------------------------------------------------------------------------
# Primitive draws
# ----------------------------------------------------------------------------

def philox(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, np.uint32)
    k = np.ascontiguousarray(key, np.uint32)
    out = np.zeros(4, np.uint32)
    lib().synth_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def normal_f32(seed: int, name: str, count: int, std: float = 1.0, start: int = 0) -> np.ndarray:
    out = np.empty(count, np.float32)
    lib().synth_normal_f32(seed, name.encode(), start, count, std, _p(out))
    return out


def normal_bf16(seed: int, name: str, count: int, std: float = 1.0, start: int = 0) -> np.ndarray:
    out = np.empty(count, np.uint16)
    lib().synth_normal_bf16(seed, name.encode(), start, count, std, _p(out))
    return out


def uniform_f32(seed: int, name: str, count: int, lo: float = 0.0, hi: float = 1.0, start: int = 0) -> np.ndarray:
    out = np.empty(count, np.float32)
    lib().synth_uniform_f32(seed, name.encode(), start, count, lo, hi, _p(out))
    return out


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().synth_f32_to_bf16(_p(a), _p(out), a.size)
    return out


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32)


def mxfp4_quantize(v: np.ndarray) -> np.ndarray:
    """[rows][K] float32 -> one MXFP4 buffer: packed [rows][K/2] then scales [rows][K/32]."""
    v = np.ascontiguousarray(v, np.float32)
    rows, K = v.shape
    assert K % 32 == 0
    buf = np.empty(rows * K // 2 + rows * K // 32, np.uint8)
    lib().synth_mxfp4_quantize(_p(v), rows, K, _p(buf), _p(buf[rows * K // 2:]))
    return buf


def normal_rows(seed: int, name: str, rows: int, K: int, std: float, bf16: bool = True,
                mxfp4: bool = False):
    """All rows of a [rows][K] N(0,std) tensor: (bf16 bits or None, MXFP4 buffer or None)."""
    b = np.empty((rows, K), np.uint16) if bf16 else None
    m = np.empty(rows * K // 2 + rows * K // 32, np.uint8) if mxfp4 else None
    lib().synth_normal_rows(seed, name.encode(), 0, rows, K, std, _p(b), _p(m),
                            None if m is None else _p(m[rows * K // 2:]))
    return b, m


def zipf_bias(n: int, s: float = 1.2, scale: float = 1.5) -> np.ndarray:
    """Selection bias b_e = scale * ln(w_rank), expert e at Zipf rank e+1 and
    w_r = r^-s / sum_{j<=n} j^-s (natural log)."""
    H = math.fsum(j ** -s for j in range(1, n + 1))
    return np.array([scale * math.log((e + 1) ** -s / H) for e in range(n)], np.float32)


# ----------------------------------------------------------------------------
# Workload presets
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Preset:
    name: str
    T: int
    d: int
    L: int              # latent width; 0 = experts read the full-width input
    n: int
    k: int
    F: int
    kind: str           # "relu2" | "swiglu3"
    act: str            # "f32" | "bf16"
    weights: str        # "f32" | "bf16" | "mxfp4"
    router_w: str       # "f32" | "bf16"
    in_norm: str = "none"          # "none" | "centered" | "input_scaled"
    expert_norm: str = "none"
    res_gate: str = "none"         # "none" | "linear" | "muse"
    eps_in: float = 1e-5
    eps_expert: float = 1e-6
    layer_seed: int = 1
    input_seed: int = 1
    router_bias: str = "none"      # "none" | "zipf" | "normal" | "normal_wide" (correction biases, see gains())
    chunks: int = 1
    w_std: float = 0.02            # latent layers; c0 uses 1/sqrt(fan_in)
    bias_in_weights: int = 0
    interm: str = "f16"            # dtype a device keeps z, SwiGLU output and m in: "f16" | "bf16"
    router_fn: str = "softmax"     # "softmax" | "sigmoid"
    out_mult: float = 1.0          # sigmoid router: logit multiplier
    routed_scale: float = 1.0      # sigmoid router: routed scaling factor
    latent_norm: str = "none"      # norm of the latent z before the experts: "none" | "centered"
    eps_latent: float = 1e-5
    out_norm: str = "none"         # norm of the branch output: "none" | "centered" | "input_scaled"
    eps_out: float = 1e-5
    res_tau: float = 0.3           # Muse residual gate temperature and floor
    res_floor: float = 1e-3
    act_quant: str = "none"        # "none" | "mxfp8": the expert GEMMs read MXFP8 activations

    @property
    def chunk_T(self) -> int:
        return self.T // self.chunks

    def cfg(self) -> dict:
        return dataclasses.asdict(self)


def _latent(name, T, input_seed, **kw):
    return Preset(name=name, T=T, d=8192, L=4096, n=256, k=8, F=4096, kind="swiglu3", act="bf16",
                  weights=kw.pop("weights", "bf16"), router_w="bf16", expert_norm="input_scaled",
                  res_gate="linear", eps_expert=1e-6, layer_seed=1, input_seed=input_seed, **kw)


PRESETS = {
    "c0": Preset(name="c0", T=64, d=64, L=0, n=8, k=2, F=128, kind="relu2", act="f32", weights="f32",
                 router_w="f32", layer_seed=0, input_seed=0),
    "c1": _latent("c1", 64, 1),
    "c2": _latent("c2", 8192, 2),
    "c3": _latent("c3", 16384, 3, router_bias="zipf"),
    "c4c": _latent("c4c", 32768, 4, weights="mxfp4", in_norm="centered", chunks=4),
    "c4i": _latent("c4i", 32768, 4, weights="mxfp4", in_norm="input_scaled", chunks=4),
}


def muse(name: str = "muse", T: int = 8192, input_seed: int = 5, **kw) -> Preset:
    """The latent layer with the Muse sublayer around it: centered input
    norm, sigmoid router with a small correction bias, latent pre-norm,
    input-scaled expert and FFN output norms (block epsilon 1e-5), and the
    alpha/beta residual gate."""
    base = dict(weights="bf16", in_norm="centered", eps_in=1e-5, router_fn="sigmoid", router_bias="normal",
                latent_norm="centered", out_norm="input_scaled", res_gate="muse")
    base.update(kw)
    return dataclasses.replace(_latent(name, T, input_seed), eps_expert=1e-5, **base)


PRESETS["m1"] = muse("m1", 64, 6)      # decode batch
PRESETS["m2"] = muse("m2", 8192, 5)    # prefill batch
# the c4 workload (MXFP4 weights, centered input norm, 4 chunks of 8192) with MXFP8 activations at the
# expert GEMMs (the scaled fp8 x fp4 MFMA)
PRESETS["c4q"] = dataclasses.replace(PRESETS["c4c"], name="c4q", act_quant="mxfp8")
# the decode batch (c1) on the MXFP4 forms of the same weights: the 4-bit checkpoint at decode
PRESETS["c1m"] = dataclasses.replace(PRESETS["c1"], name="c1m", weights="mxfp4")


def small(name: str = "small", T: int = 77, d: int = 512, L: int = 256, F: int = 256, n: int = 16,
          k: int = 4, **kw) -> Preset:
    """A reduced latent layer with the same recipe (several tiles, ragged T)."""
    base = dict(name=name, T=T, d=d, L=L, n=n, k=k, F=F, kind="swiglu3", act="bf16", weights="bf16",
                router_w="bf16", expert_norm="input_scaled", res_gate="linear", layer_seed=11,
                input_seed=12)
    base.update(kw)
    return Preset(**base)


def _w1_shape(p: Preset):
    if p.kind == "swiglu3":
        return (p.n, 2 * p.F, p.L if p.L else p.d)
    return (p.n, p.F, p.L if p.L else p.d)


def _w2_shape(p: Preset):
    return (p.n, p.L if p.L else p.d, p.F)


def layer_params(p: Preset, formats=None) -> dict:
    """Layer parameters of a preset as host arrays (stored bits).

    formats: which stored forms of the big weights to make: a subset of
    {"f32", "bf16", "mxfp4"}; defaults to the preset's own.  Keys:
    router_w, down_w, w1, w2, up_w (for the preset's format), and when
    several formats are asked for, also "<key>@<fmt>".  Gains: gamma_ex,
    gate, gamma_in (float32), bias (float32 or absent).
    """
    formats = tuple(formats or (p.weights,))
    s = p.layer_seed
    out = {}
    Kin = p.L if p.L else p.d

    def std_for(fan_in):
        return p.w_std if p.L else 1.0 / math.sqrt(fan_in)

    # router: always bf16 or f32 as the preset says
    if p.router_w == "f32":
        out["router_w"] = normal_f32(s, "router_w", p.n * p.d, std_for(p.d)).reshape(p.n, p.d)
    else:
        out["router_w"] = normal_bf16(s, "router_w", p.n * p.d, std_for(p.d)).reshape(p.n, p.d)

    mats = []
    if p.L:
        mats.append(("down_w", "down_w", (p.L, p.d), std_for(p.d)))
        mats.append(("up_w", "up_w", (p.d, p.L), std_for(p.L)))
    w1s, w2s = _w1_shape(p), _w2_shape(p)
    mats.append(("w1", "expert_w1", w1s, std_for(w1s[2])))
    mats.append(("w2", "expert_w2", w2s, std_for(w2s[2])))
    for key, tname, shape, std in mats:
        rows = int(np.prod(shape[:-1]))
        K = shape[-1]
        forms = {}
        if "f32" in formats:
            forms["f32"] = normal_f32(s, tname, rows * K, std).reshape(shape)
        need_b, need_m = "bf16" in formats, "mxfp4" in formats
        if need_b or need_m:
            b, m = normal_rows(s, tname, rows, K, std, bf16=need_b, mxfp4=need_m)
            if need_b:
                forms["bf16"] = b.reshape(shape)
            if need_m:
                forms["mxfp4"] = m
        for f, a in forms.items():
            if f == p.weights:
                out[key] = a
            if len(formats) > 1:
                out[key + "@" + f] = a
    out.update(gains(p))
    return out


def gains(p: Preset) -> dict:
    """The layer's small fp32 parameter vectors: gamma_ex, gate, gamma_in,
    gamma_lat, gamma_out and bias, each present when its stage is on."""
    s = p.layer_seed
    Kin = p.L if p.L else p.d
    out = {}
    if p.expert_norm != "none":
        out["gamma_ex"] = normal_f32(s, "gamma_expert", Kin, 0.02)
    if p.res_gate == "linear":
        out["gate"] = uniform_f32(s, "res_gate", p.d, 0.0, 1.0)
    elif p.res_gate == "muse":
        # spans the floor: alpha is clamped where g > 2.28 (tau 0.3, floor 1e-3)
        out["gate"] = uniform_f32(s, "res_gate_muse", p.d, -3.0, 3.0)
    if p.in_norm != "none":
        out["gamma_in"] = normal_f32(s, "gamma_in", p.d, 0.02)
    if p.latent_norm != "none":
        out["gamma_lat"] = normal_f32(s, "gamma_latent", p.L, 0.02)
    if p.out_norm != "none":
        out["gamma_out"] = normal_f32(s, "gamma_out", p.d, 0.02)
    if p.router_bias == "zipf":
        out["bias"] = zipf_bias(p.n)
    elif p.router_bias in ("normal", "normal_wide"):
        # A correction bias for sigmoid scores.  "normal" (std 0.002) is of the
        # order of the gaps between a token's top sigmoid scores at the full
        # shape: it changes the expert set of ~30% of the tokens while the
        # load stays about as balanced as without it (the bias exists to
        # balance load).  "normal_wide" (std 0.05) swamps those gaps: a few
        # experts take most tokens (a skewed-load stress case).
        std = 0.002 if p.router_bias == "normal" else 0.05
        out["bias"] = normal_f32(s, "router_bias", p.n, std)
    return out


def inputs(p: Preset, chunk: int | None = None) -> np.ndarray:
    """x for the whole preset (chunk None) or for one chunk: [rows][d] stored bits."""
    T = p.T if chunk is None else p.chunk_T
    start = 0 if chunk is None else chunk * p.chunk_T * p.d
    if p.act == "f32":
        return normal_f32(p.input_seed, "x", T * p.d, 1.0, start).reshape(T, p.d)
    return normal_bf16(p.input_seed, "x", T * p.d, 1.0, start).reshape(T, p.d)


def sample_tokens(T: int, count: int, seed: int = 1234) -> np.ndarray:
    """A sorted seeded subset of token ids (all of them when count >= T)."""
    if count >= T:
        return np.arange(T, dtype=np.int64)
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(T, size=count, replace=False)).astype(np.int64)
