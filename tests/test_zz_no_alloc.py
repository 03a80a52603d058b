"""moe_layer_forward_static (the entry point that allocates nothing and runs
on the library's static scratch) against moe_layer_forward with a caller
workspace: the same kernels, so every output and inspected intermediate is
identical bit for bit.  Two calls in a row on one device, the second on a
smaller batch, so it runs over the first call's leftovers in the scratch."""
import ctypes

import numpy as np
import pytest
import torch

import sparse_mixture_experts_router_amd as moe
import synthetic
from gpu_helpers import DeviceLayer, desc_of, run, say, to_dev

pytestmark = pytest.mark.gpu


def run_static(layer: DeviceLayer, x: np.ndarray) -> dict:
    """One call of moe_layer_forward_static through the C ABI, with the same
    inspection outputs as gpu_helpers.run."""
    p = layer.p
    T = x.shape[0]
    xd = to_dev(x)
    out = torch.empty((T, p.d), dtype=torch.float32, device="cuda")
    D = {"topk_idx": torch.empty((T, p.k), dtype=torch.int32, device="cuda"),
         "topk_w": torch.empty((T, p.k), dtype=torch.float32, device="cuda"),
         "expert_counts": torch.empty(p.n, dtype=torch.int32, device="cuda"),
         "expert_offsets": torch.empty(p.n + 1, dtype=torch.int32, device="cuda"),
         "perm_tok": torch.empty(T * p.k, dtype=torch.int32, device="cuda"),
         "perm_slot": torch.empty(T * p.k, dtype=torch.int32, device="cuda"),
         "y": torch.empty((T, p.d), dtype=torch.float32, device="cuda"),
         "pos": torch.empty((T, p.k), dtype=torch.int32, device="cuda"),
         "logits": torch.empty((T, p.n), dtype=torch.float32, device="cuda"),
         "u": torch.empty((T, p.d), dtype=torch.int16, device="cuda")}
    dv = layer.dev
    moe.moe_layer_forward_static(desc_of(p, T), xd, dv["router_w"], dv.get("down_w"), dv["w1"], dv["w2"],
                                 dv.get("up_w"), layer.gains(), out, dbg=D)
    torch.cuda.synchronize()
    res = {"out": out.cpu().numpy()}
    for k_, v in D.items():
        a = v.cpu().numpy()
        res[k_] = a.view(np.uint16) if a.dtype == np.int16 else a
    return res


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


@pytest.mark.parametrize("name,kw,T1,T2", [
    # ~75 rows per expert on the first call: tiled expert GEMMs; streamed ones on the second
    ("static_tiles", dict(d=1024, L=512, F=512, n=16, k=4), 300, 45),
    # the Muse sublayer (input norm, sigmoid router, latent pre-norm, output norm, alpha/beta gate)
    ("static_muse", dict(d=1024, L=512, F=512, n=32, k=4, in_norm="centered", router_fn="sigmoid",
                         router_bias="normal", latent_norm="centered", out_norm="input_scaled", res_gate="muse",
                         eps_expert=1e-5), 200, 17),
])
def test_static_scratch_matches_workspace_forward(name, kw, T1, T2):
    p = synthetic.small(name=name, T=T1, **kw)
    layer = DeviceLayer(p)
    x = synthetic.inputs(p)
    for T in (T1, T2):
        assert moe.moe_workspace_bytes(desc_of(p, T)) <= moe.MOE_STATIC_SCRATCH_BYTES
        say("%s: T=%d, static scratch vs caller workspace" % (name, T))
        got = run_static(layer, x[:T])
        ref = run(layer, x[:T], stages=False)
        for key in ref:
            np.testing.assert_array_equal(got[key], ref[key], err_msg="%s T=%d %s" % (name, T, key))


def test_static_scratch_at_the_layer_shape_decode_batch():
    # the 816B-A42B layer shape at a decode batch (T=64), then a smaller one, on a reduced expert count
    # (n=16, k=8: the real d, L, F and top-k, without the 24 GB of the full expert set)
    p = synthetic.small(name="static_wide", T=64, d=8192, L=4096, F=4096, n=16, k=8)
    layer = DeviceLayer(p)
    x = synthetic.inputs(p)
    for T in (64, 9):
        got = run_static(layer, x[:T])
        ref = run(layer, x[:T], stages=False)
        for key in ref:
            np.testing.assert_array_equal(got[key], ref[key], err_msg="T=%d %s" % (T, key))


def test_static_scratch_rejects_oversized_batches_before_launching():
    p = synthetic.PRESETS["c1"]
    T = 4096
    d = desc_of(p, T)
    assert moe.moe_workspace_bytes(d) > moe.MOE_STATIC_SCRATCH_BYTES
    fake = ctypes.c_void_p(256)  # never dereferenced: the size check comes first
    g = moe.moe_gains()
    rc = moe.lib().moe_layer_forward_static(ctypes.byref(d), fake, fake, fake, fake, fake, fake, ctypes.byref(g),
                                            fake, None, None)
    assert rc == moe.MOE_ERR_STATIC_SCRATCH_TOO_SMALL
    assert "static scratch" in moe.moe_error_string(rc)
