"""MI355X latent sparse mixture-of-experts layer: Python binding.

Thin ctypes marshalling over the C ABI of ``include/moe.h`` (library
``libmoe_mi355x.so`` built from ``csrc/`` for gfx950).  Every step of the
layer runs in that library's HIP kernels; this module only checks tensors and
passes device pointers.  There is no fallback: if the library is missing the
import of any entry point raises.

Names follow the C ABI: ``moe_layer_forward``, ``moe_layer_forward_static``, ``moe_workspace_bytes``,
``moe_validate``, ``moe_error_string``, ``moe_router_topk``,
``moe_router_workspace_bytes``, ``moe_permute``, ``moe_convert_bf16_to_f16``,
``moe_hbm_copy``.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_ERR_STATIC_SCRATCH_TOO_SMALL = -5
MOE_STATIC_SCRATCH_BYTES = 64 << 20  # the static scratch of moe_layer_forward_static (include/moe.h)
DT = {"f32": 0, "bf16": 1, "mxfp4": 2, "f16": 3}
NORM = {"none": 0, "centered": 1, "input_scaled": 2}
KIND = {"relu2": 0, "swiglu3": 1}
RES = {"none": 0, "linear": 1, "muse": 2}
ROUTER = {"softmax": 0, "sigmoid": 1}
ACT_QUANT = {"none": 0, "mxfp8": 1}
STAGES = ["in_norm", "router", "topk", "permute", "down", "gemm1", "gemm2", "combine", "up", "resgate"]
GAINS = ("router_bias", "gamma_in", "gamma_expert", "res_gate", "gamma_latent", "gamma_out")


class MoeError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        super().__init__("%s: %s (%d)" % (what or "moe", moe_error_string(code), code))
        self.code = code


class moe_desc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d_model", ctypes.c_int64), ("d_latent", ctypes.c_int64),
                ("n_experts", ctypes.c_int64), ("top_k", ctypes.c_int64), ("d_ff", ctypes.c_int64),
                ("expert_kind", ctypes.c_int32), ("act_dtype", ctypes.c_int32), ("router_dtype", ctypes.c_int32),
                ("weight_dtype", ctypes.c_int32), ("in_norm", ctypes.c_int32), ("expert_norm", ctypes.c_int32),
                ("res_gate", ctypes.c_int32), ("bias_in_weights", ctypes.c_int32), ("eps_in", ctypes.c_float),
                ("eps_expert", ctypes.c_float), ("interm_dtype", ctypes.c_int32), ("router_fn", ctypes.c_int32),
                ("router_out_mult", ctypes.c_float), ("routed_scale", ctypes.c_float),
                ("latent_norm", ctypes.c_int32), ("eps_latent", ctypes.c_float), ("out_norm", ctypes.c_int32),
                ("eps_out", ctypes.c_float), ("res_tau", ctypes.c_float), ("res_floor", ctypes.c_float),
                ("act_quant", ctypes.c_int32)]


class moe_gains(ctypes.Structure):
    _fields_ = [(nm, ctypes.c_void_p) for nm in GAINS]


class moe_debug(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p), ("expert_counts", ctypes.c_void_p),
                ("expert_offsets", ctypes.c_void_p), ("perm_tok", ctypes.c_void_p), ("perm_slot", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("pos", ctypes.c_void_p), ("z", ctypes.c_void_p), ("act", ctypes.c_void_p),
                ("S", ctypes.c_void_p), ("ssq", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("stage_events", ctypes.c_void_p), ("logits", ctypes.c_void_p), ("u", ctypes.c_void_p),
                ("zq", ctypes.c_void_p), ("actq", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmoe_mi355x.so is not built; run __graft_entry__.build() "
                              "(hipcc --offload-arch=gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        L.moe_error_string.argtypes = [ctypes.c_int]
        L.moe_error_string.restype = ctypes.c_char_p
        L.moe_validate.argtypes = [ctypes.POINTER(moe_desc)]
        L.moe_workspace_bytes.argtypes = [ctypes.POINTER(moe_desc)]
        L.moe_workspace_bytes.restype = sz
        L.moe_layer_forward.argtypes = [ctypes.POINTER(moe_desc), vp, vp, vp, vp, vp, vp, ctypes.POINTER(moe_gains),
                                        vp, vp, sz, ctypes.POINTER(moe_debug), vp]
        L.moe_layer_forward_static.argtypes = [ctypes.POINTER(moe_desc), vp, vp, vp, vp, vp, vp,
                                               ctypes.POINTER(moe_gains), vp, ctypes.POINTER(moe_debug), vp]
        L.moe_router_workspace_bytes.argtypes = [ctypes.POINTER(moe_desc)]
        L.moe_router_workspace_bytes.restype = sz
        L.moe_router_topk.argtypes = [ctypes.POINTER(moe_desc), vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_permute.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
        L.moe_hbm_copy.argtypes = [vp, vp, sz, vp]
        L.moe_convert_bf16_to_f16.argtypes = [vp, vp, i64, vp]
        _lib = L
    return _lib


EXPORTED = ["moe_error_string", "moe_validate", "moe_workspace_bytes", "moe_layer_forward", "moe_layer_forward_static",
            "moe_router_workspace_bytes", "moe_router_topk", "moe_permute", "moe_convert_bf16_to_f16", "moe_hbm_copy"]


def make_desc(T, d_model, d_latent, n_experts, top_k, d_ff, expert_kind="swiglu3", act="bf16", router="bf16",
              weights="bf16", in_norm="none", expert_norm="none", res_gate="none", bias_in_weights=0,
              eps_in=1e-5, eps_expert=1e-6, interm="f16", router_fn="softmax", out_mult=1.0, routed_scale=1.0,
              latent_norm="none", eps_latent=1e-5, out_norm="none", eps_out=1e-5, res_tau=0.3,
              res_floor=1e-3, act_quant="none") -> moe_desc:
    return moe_desc(T=T, d_model=d_model, d_latent=d_latent, n_experts=n_experts, top_k=top_k, d_ff=d_ff,
                    expert_kind=KIND[expert_kind], act_dtype=DT[act], router_dtype=DT[router],
                    weight_dtype=DT[weights], in_norm=NORM[in_norm], expert_norm=NORM[expert_norm],
                    res_gate=RES[res_gate], bias_in_weights=int(bias_in_weights), eps_in=eps_in,
                    eps_expert=eps_expert, interm_dtype=DT[interm], router_fn=ROUTER[router_fn],
                    router_out_mult=out_mult, routed_scale=routed_scale, latent_norm=NORM[latent_norm],
                    eps_latent=eps_latent, out_norm=NORM[out_norm], eps_out=eps_out, res_tau=res_tau,
                    res_floor=res_floor, act_quant=ACT_QUANT[act_quant])


def moe_error_string(code: int) -> str:
    return lib().moe_error_string(int(code)).decode()


def moe_validate(desc: moe_desc) -> int:
    return lib().moe_validate(ctypes.byref(desc))


def moe_workspace_bytes(desc: moe_desc) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(desc))


def moe_router_workspace_bytes(desc: moe_desc) -> int:
    return lib().moe_router_workspace_bytes(ctypes.byref(desc))


def _ptr(t, what: str, nbytes: int | None = None):
    """Device pointer of a contiguous CUDA tensor (or None / a raw int)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % what)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % what)
    if nbytes is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError("%s holds %d bytes, needs %d" % (what, t.numel() * t.element_size(), nbytes))
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _scratch(nbytes: int, device, stream):
    """A uint8 device buffer for a call enqueued on `stream`.  It comes from
    torch's caching allocator on the current stream; when the call goes to
    another torch stream the buffer is recorded on that stream, so the
    allocator does not hand its memory out again before the call's kernels
    are done.  A raw stream handle other than the current stream cannot be
    recorded: such calls must pass their own buffer."""
    import torch
    buf = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if stream is not None:
        cur = torch.cuda.current_stream(device)
        if isinstance(stream, int):
            if stream != cur.cuda_stream:
                raise ValueError("a call on a raw stream handle other than torch's current stream needs an "
                                 "explicit workspace")
        elif stream != cur:
            buf.record_stream(stream)
    return buf


def _wbytes(desc: moe_desc, rows: int, K: int) -> int:
    if desc.weight_dtype == DT["mxfp4"]:
        return rows * K // 2 + rows * K // 32
    return rows * K * (4 if desc.weight_dtype == DT["f32"] else 2)


def moe_layer_forward(desc: moe_desc, x, router_w, down_w, expert_w1, expert_w2, up_w, gains: dict | None, out,
                      workspace=None, dbg: dict | None = None, stream=None):
    """Enqueue one layer forward on `stream` (default: torch's current stream).

    gains: dict of device fp32 tensors under router_bias, gamma_in,
    gamma_expert, res_gate, gamma_latent, gamma_out (absent = NULL).  dbg:
    dict of device tensors under the moe_debug field names, plus optionally
    "stage_events" (an int address of 2 * len(STAGES) hipEvent_t).  workspace: uint8 device tensor of at least
    moe_workspace_bytes(desc) bytes (allocated here when None, and then kept
    from reuse until the call's kernels on `stream` are done).
    """
    import torch
    T, d, L, n, k, F = desc.T, desc.d_model, desc.d_latent, desc.n_experts, desc.top_k, desc.d_ff
    ab = 4 if desc.act_dtype == DT["f32"] else 2
    rb = 4 if desc.router_dtype == DT["f32"] else 2
    Din = L if L else d
    rows1 = n * (2 * F if desc.expert_kind == KIND["swiglu3"] else F)
    need = moe_workspace_bytes(desc)
    if workspace is None:
        workspace = _scratch(need, x.device, stream)
    g = moe_gains()
    for nm in GAINS:
        v = (gains or {}).get(nm)
        if v is not None and v.dtype != torch.float32:
            raise ValueError("gain %s must be float32" % nm)
        setattr(g, nm, _ptr(v, nm))
    dd = None
    if dbg:
        dd = moe_debug()
        for nm, _ in moe_debug._fields_:
            v = dbg.get(nm)
            setattr(dd, nm, _ptr(v, nm) if nm != "stage_events" else v)
    rc = lib().moe_layer_forward(
        ctypes.byref(desc), _ptr(x, "x", T * d * ab), _ptr(router_w, "router_w", n * d * rb),
        _ptr(down_w, "down_w", _wbytes(desc, L, d) if L else None), _ptr(expert_w1, "expert_w1", _wbytes(desc, rows1, Din)),
        _ptr(expert_w2, "expert_w2", _wbytes(desc, n * Din, F)), _ptr(up_w, "up_w", _wbytes(desc, d, L) if L else None),
        ctypes.byref(g), _ptr(out, "out", T * d * 4), _ptr(workspace, "workspace"),
        workspace.numel() if not isinstance(workspace, int) else need, ctypes.byref(dd) if dd else None,
        _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_layer_forward")
    return out


def moe_layer_forward_static(desc: moe_desc, x, router_w, down_w, expert_w1, expert_w2, up_w, gains: dict | None,
                             out, dbg: dict | None = None, stream=None):
    """moe_layer_forward on the library's static scratch: no workspace and
    no allocation (batches up to MOE_STATIC_SCRATCH_BYTES of workspace)."""
    import torch
    T, d, L, n, F = desc.T, desc.d_model, desc.d_latent, desc.n_experts, desc.d_ff
    ab = 4 if desc.act_dtype == DT["f32"] else 2
    rb = 4 if desc.router_dtype == DT["f32"] else 2
    Din = L if L else d
    rows1 = n * (2 * F if desc.expert_kind == KIND["swiglu3"] else F)
    g = moe_gains()
    for nm in GAINS:
        v = (gains or {}).get(nm)
        if v is not None and v.dtype != torch.float32:
            raise ValueError("gain %s must be float32" % nm)
        setattr(g, nm, _ptr(v, nm))
    dd = None
    if dbg:
        dd = moe_debug()
        for nm, _ in moe_debug._fields_:
            v = dbg.get(nm)
            setattr(dd, nm, _ptr(v, nm) if nm != "stage_events" else v)
    rc = lib().moe_layer_forward_static(
        ctypes.byref(desc), _ptr(x, "x", T * d * ab), _ptr(router_w, "router_w", n * d * rb),
        _ptr(down_w, "down_w", _wbytes(desc, L, d) if L else None), _ptr(expert_w1, "expert_w1", _wbytes(desc, rows1, Din)),
        _ptr(expert_w2, "expert_w2", _wbytes(desc, n * Din, F)), _ptr(up_w, "up_w", _wbytes(desc, d, L) if L else None),
        ctypes.byref(g), _ptr(out, "out", T * d * 4), ctypes.byref(dd) if dd else None, _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_layer_forward_static")
    return out


def moe_router_topk(desc: moe_desc, u, router_w, router_bias, topk_idx, topk_w, logits=None, workspace=None,
                    stream=None):
    if logits is None and workspace is None:
        workspace = _scratch(moe_router_workspace_bytes(desc), u.device, stream)
    rc = lib().moe_router_topk(ctypes.byref(desc), _ptr(u, "u"), _ptr(router_w, "router_w"),
                               _ptr(router_bias, "router_bias"), _ptr(topk_idx, "topk_idx"), _ptr(topk_w, "topk_w"),
                               _ptr(logits, "logits"), _ptr(workspace, "workspace"),
                               0 if workspace is None else workspace.numel(), _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_router_topk")


def moe_permute(T, k, n, topk_idx, counts, offsets, perm_tok, perm_slot, pos, stream=None):
    rc = lib().moe_permute(T, k, n, _ptr(topk_idx, "topk_idx"), _ptr(counts, "counts"), _ptr(offsets, "offsets"),
                           _ptr(perm_tok, "perm_tok"), _ptr(perm_slot, "perm_slot"), _ptr(pos, "pos"),
                           _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_permute")


def moe_convert_bf16_to_f16(src, dst, count: int, stream=None):
    """bf16 -> fp16 (round to nearest even) of `count` values; dst may be src."""
    rc = lib().moe_convert_bf16_to_f16(_ptr(src, "src", 2 * count), _ptr(dst, "dst", 2 * count), count,
                                       _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_convert_bf16_to_f16")


def moe_hbm_copy(dst, src, nbytes: int, stream=None):
    rc = lib().moe_hbm_copy(_ptr(dst, "dst", nbytes), _ptr(src, "src", nbytes), nbytes, _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_hbm_copy")


# ---------------------------------------------------------------------------
# HIP events for per-stage timing on the library's stream
# ---------------------------------------------------------------------------

class StageEvents:
    """2 * MOE_NUM_STAGES hipEvent_t, for moe_debug.stage_events."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventQuery.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipGetLastError.restype = ctypes.c_int
        n = 2 * len(STAGES)
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.arr[i] = ev
        self.recorded = set()

    @property
    def address(self) -> int:
        return ctypes.addressof(self.arr)

    def elapsed_ms(self, stage: str):
        """Milliseconds of a stage of the last recorded call (None if it did
        not run).  A failed query leaves HIP's last-error state set, which the
        next framework call would report as its own failure, so it is cleared
        here."""
        s = STAGES.index(stage)
        a, b = self.arr[2 * s], self.arr[2 * s + 1]
        ms = ctypes.c_float()
        if (self.hip.hipEventQuery(a) != 0 or self.hip.hipEventQuery(b) != 0
                or self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0):
            self.hip.hipGetLastError()
            return None
        return ms.value

    def close(self):
        for i in range(len(self.arr)):
            if self.arr[i]:
                self.hip.hipEventDestroy(self.arr[i])
                self.arr[i] = None
