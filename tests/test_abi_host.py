"""The C-ABI library loads and exports every symbol include/moe.h declares;
host-only entry points (validation, workspace sizing, error strings) work
without a GPU.  No compute call is made here."""
import ctypes
import dataclasses
import os
import re

import pytest

import sparse_mixture_experts_router_amd as moe
import synthetic
from conftest import preset_desc

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


desc_of = preset_desc


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
    ("res_gate", 3, moe.MOE_ERR_INVALID_ARG),
    ("router_fn", 2, moe.MOE_ERR_INVALID_ARG),
    ("latent_norm", 3, moe.MOE_ERR_INVALID_ARG),
    ("latent_norm", 2, moe.MOE_ERR_UNSUPPORTED),
    ("out_norm", 3, moe.MOE_ERR_INVALID_ARG),
    ("eps_expert", -1.0, moe.MOE_ERR_INVALID_ARG),
    ("d_model", 8192 + 64, moe.MOE_ERR_UNSUPPORTED),
    ("d_latent", 0, moe.MOE_ERR_UNSUPPORTED),
    ("weight_dtype", 0, moe.MOE_ERR_UNSUPPORTED),
    ("n_experts", 250, moe.MOE_ERR_UNSUPPORTED),
    ("T", (1 << 30) // 4096, moe.MOE_ERR_UNSUPPORTED),   # latent z of 2 GiB: past 32-bit row offsets
])
def test_validation_errors(field, value, code):
    d = desc_of(synthetic.PRESETS["c1"])
    setattr(d, field, value)
    assert moe.moe_validate(d) == code
    assert moe.moe_workspace_bytes(d) == 0


def test_largest_batch_of_the_latent_path_validates():
    d = desc_of(synthetic.PRESETS["c1"])
    d.T = (1 << 30) // 4096 - 1
    assert moe.moe_validate(d) == moe.MOE_OK


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


@pytest.mark.parametrize("changes,code", [
    ({"bias_in_weights": 1}, moe.MOE_ERR_INVALID_ARG),              # the sigmoid's bias selects only
    ({"router_out_mult": float("inf")}, moe.MOE_ERR_INVALID_ARG),
    ({"routed_scale": float("nan")}, moe.MOE_ERR_INVALID_ARG),
    ({"res_tau": 0.0}, moe.MOE_ERR_INVALID_ARG),
    ({"res_tau": float("inf")}, moe.MOE_ERR_INVALID_ARG),
    ({"res_floor": -1e-3}, moe.MOE_ERR_INVALID_ARG),
    ({"eps_out": -1.0}, moe.MOE_ERR_INVALID_ARG),
    ({"eps_latent": -1.0}, moe.MOE_ERR_INVALID_ARG),
    ({"d_model": 8192 + 512}, moe.MOE_ERR_UNSUPPORTED),             # output norm rows hold <= 8192 values
    ({"router_out_mult": -2.0, "routed_scale": 0.0, "res_floor": 0.0}, moe.MOE_OK),
])
def test_muse_descriptor_validation(changes, code):
    d = desc_of(synthetic.PRESETS["m1"])
    assert moe.moe_validate(d) == moe.MOE_OK
    for k_, v in changes.items():
        setattr(d, k_, v)
    assert moe.moe_validate(d) == code


def test_muse_stages_on_the_fp32_path_and_workspace():
    c0 = synthetic.PRESETS["c0"]
    d = desc_of(c0)
    d.router_fn = moe.ROUTER["sigmoid"]             # the router kernel is shared: allowed
    assert moe.moe_validate(d) == moe.MOE_OK
    for field, v in (("out_norm", moe.NORM["input_scaled"]), ("res_gate", moe.RES["muse"])):
        e = desc_of(c0)
        setattr(e, field, v)
        assert moe.moe_validate(e) == moe.MOE_ERR_UNSUPPORTED, field
    e = desc_of(c0)
    e.latent_norm = moe.NORM["centered"]            # no latent to normalise
    assert moe.moe_validate(e) == moe.MOE_ERR_INVALID_ARG
    # the output norm's bf16 rows and partial sums take T * d * (2 + 4/16) more bytes
    m1 = synthetic.PRESETS["m1"]
    a = moe.moe_workspace_bytes(desc_of(m1))
    b = moe.moe_workspace_bytes(desc_of(dataclasses.replace(m1, out_norm="none")))
    assert a - b >= m1.T * m1.d * (2 + 4 / 16)


def test_muse_forward_needs_its_gate_vector():
    lib = moe.lib()
    d = desc_of(synthetic.PRESETS["m1"])
    g = moe.moe_gains()
    fake = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    rc = lib.moe_layer_forward(ctypes.byref(d), fake, fake, fake, fake, fake, fake, ctypes.byref(g), fake, fake,
                               1 << 40, None, None)
    assert rc == moe.MOE_ERR_INVALID_ARG
    assert ctypes.sizeof(moe.moe_desc) == 136 and ctypes.sizeof(moe.moe_gains) == 48


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


def test_binding_structs_match_the_header(tmp_path):
    # sizeof and every field offset of the three C structs, compiled from include/moe.h,
    # against the ctypes structures the binding passes
    structs = {"moe_desc": moe.moe_desc, "moe_gains": moe.moe_gains, "moe_debug": moe.moe_debug}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "moe.h"', "int main(void) {"]
    for sn, cls in structs.items():
        lines.append('printf("%s sizeof %%zu\\n", sizeof(%s));' % (sn, sn))
        for fn, _ in cls._fields_:
            lines.append('printf("%s %s %%zu\\n", offsetof(%s, %s));' % (sn, fn, sn, fn))
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    import subprocess
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = {}
    for line in subprocess.check_output([str(exe)], text=True).splitlines():
        sn, fn, v = line.split()
        got[(sn, fn)] = int(v)
    for sn, cls in structs.items():
        assert got[(sn, "sizeof")] == ctypes.sizeof(cls), sn
        for fn, _ in cls._fields_:
            assert got[(sn, fn)] == getattr(cls, fn).offset, (sn, fn)


def test_mxfp8_activations_need_mxfp4_weights():
    p = dataclasses.replace(synthetic.PRESETS["c4q"], name="q8_bf16w", weights="bf16")
    assert moe.moe_validate(desc_of(p)) == moe.MOE_ERR_UNSUPPORTED
    assert moe.moe_validate(desc_of(synthetic.PRESETS["c4q"])) == moe.MOE_OK
    d = desc_of(synthetic.PRESETS["c4q"])
    d.act_quant = 2
    assert moe.moe_validate(d) == moe.MOE_ERR_INVALID_ARG
    # the quantized forms of z and of the SwiGLU output: 33/32 bytes per value each
    a, b = moe.moe_workspace_bytes(desc_of(synthetic.PRESETS["c4q"])), moe.moe_workspace_bytes(
        desc_of(synthetic.PRESETS["c4c"]))
    p = synthetic.PRESETS["c4q"]
    assert a - b >= p.chunk_T * (p.L + p.k * p.F) * 33 // 32
