"""The C-ABI library loads and exports every symbol include/moe.h declares;
host-only entry points (validation, workspace sizing, error strings) work
without a GPU.  No compute call is made here."""
import ctypes
import os
import re

import pytest

import sparse_mixture_experts_router_amd as moe
import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = moe.lib()
    names = declared_functions()
    assert len(names) >= 7, names
    for nm in names:
        assert hasattr(lib, nm), nm
    assert set(moe.EXPORTED) == set(names)


def desc_of(p, T=None):
    return moe.make_desc(T if T is not None else p.chunk_T, p.d, p.L, p.n, p.k, p.F, expert_kind=p.kind, act=p.act,
                         router=p.router_w, weights=p.weights, in_norm=p.in_norm, expert_norm=p.expert_norm,
                         res_gate=p.res_gate, eps_in=p.eps_in, eps_expert=p.eps_expert)


@pytest.mark.parametrize("name", list(synthetic.PRESETS))
def test_presets_validate(name):
    d = desc_of(synthetic.PRESETS[name])
    assert moe.moe_validate(d) == moe.MOE_OK
    assert moe.moe_workspace_bytes(d) > 0


def test_workspace_grows_with_T_and_is_aligned():
    p = synthetic.PRESETS["c1"]
    a, b = moe.moe_workspace_bytes(desc_of(p, 64)), moe.moe_workspace_bytes(desc_of(p, 8192))
    assert 0 < a < b and a % 256 == 0 and b % 256 == 0
    # T = 0 is valid
    assert moe.moe_validate(desc_of(p, 0)) == moe.MOE_OK


@pytest.mark.parametrize("field,value,code", [
    ("top_k", 0, moe.MOE_ERR_INVALID_ARG),
    ("top_k", 257, moe.MOE_ERR_INVALID_ARG),
    ("n_experts", 300, moe.MOE_ERR_INVALID_ARG),
    ("T", -1, moe.MOE_ERR_INVALID_ARG),
    ("d_model", 0, moe.MOE_ERR_INVALID_ARG),
    ("act_dtype", 7, moe.MOE_ERR_INVALID_ARG),
    ("weight_dtype", 5, moe.MOE_ERR_INVALID_ARG),
    ("in_norm", 3, moe.MOE_ERR_INVALID_ARG),
    ("res_gate", 2, moe.MOE_ERR_INVALID_ARG),
    ("eps_expert", -1.0, moe.MOE_ERR_INVALID_ARG),
    ("d_model", 8192 + 64, moe.MOE_ERR_UNSUPPORTED),
    ("d_latent", 0, moe.MOE_ERR_UNSUPPORTED),
    ("weight_dtype", 0, moe.MOE_ERR_UNSUPPORTED),
    ("n_experts", 250, moe.MOE_ERR_UNSUPPORTED),
])
def test_validation_errors(field, value, code):
    d = desc_of(synthetic.PRESETS["c1"])
    setattr(d, field, value)
    assert moe.moe_validate(d) == code
    assert moe.moe_workspace_bytes(d) == 0


def test_forward_rejects_before_any_launch():
    # Errors are returned on the host before anything touches a device.
    lib = moe.lib()
    d = desc_of(synthetic.PRESETS["c1"])
    g = moe.moe_gains()
    fake = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    # NULL x
    rc = lib.moe_layer_forward(ctypes.byref(d), None, fake, fake, fake, fake, fake, ctypes.byref(g), fake, fake,
                               1 << 40, None, None)
    assert rc == moe.MOE_ERR_INVALID_ARG
    # workspace too small
    g.res_gate = 256
    rc = lib.moe_layer_forward(ctypes.byref(d), fake, fake, fake, fake, fake, fake, ctypes.byref(g), fake, fake, 16,
                               None, None)
    assert rc == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    # residual gate requested without its vector
    g.res_gate = None
    rc = lib.moe_layer_forward(ctypes.byref(d), fake, fake, fake, fake, fake, fake, ctypes.byref(g), fake, fake,
                               1 << 40, None, None)
    assert rc == moe.MOE_ERR_INVALID_ARG
    # permute stage argument checks
    assert lib.moe_permute(4, 0, 8, fake, fake, fake, fake, fake, fake, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_permute(4, 2, 8, None, fake, fake, fake, fake, fake, None) == moe.MOE_ERR_INVALID_ARG


def test_error_strings():
    assert moe.moe_error_string(0) == "ok"
    assert "workspace" in moe.moe_error_string(-3)
    assert moe.moe_error_string(-99) == "unknown status"


def test_f16_weight_format_validation():
    d = desc_of(synthetic.PRESETS["c1"])
    d.weight_dtype = moe.DT["f16"]
    assert moe.moe_validate(d) == moe.MOE_OK
    assert moe.moe_workspace_bytes(d) == moe.moe_workspace_bytes(desc_of(synthetic.PRESETS["c1"]))
    d.interm_dtype = moe.DT["bf16"]  # fp16 weights feed the fp16 GEMMs only
    assert moe.moe_validate(d) == moe.MOE_ERR_UNSUPPORTED


def test_convert_rejects_before_any_launch():
    lib = moe.lib()
    a, b = ctypes.c_void_p(4096), ctypes.c_void_p(1 << 20)  # never dereferenced
    bad = moe.MOE_ERR_INVALID_ARG
    assert lib.moe_convert_bf16_to_f16(a, b, 12, None) == bad                    # not a multiple of 8
    assert lib.moe_convert_bf16_to_f16(a, b, -8, None) == bad
    assert lib.moe_convert_bf16_to_f16(ctypes.c_void_p(4098), b, 8, None) == bad  # misaligned
    assert lib.moe_convert_bf16_to_f16(None, b, 8, None) == bad
    assert lib.moe_convert_bf16_to_f16(a, ctypes.c_void_p(4096 + 16), 64, None) == bad  # partial overlap
    assert lib.moe_convert_bf16_to_f16(None, None, 0, None) == moe.MOE_OK       # nothing to do
