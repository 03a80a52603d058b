"""GPU parity of the HIP layer against the CPU oracle at sizes the oracle
finishes in seconds (several tiles, ragged tails), through the C ABI.

Bars: routing indices and permutation bit-exact (near-ties with margin
< 1e-4 excluded), outputs within 1e-5 * RMS(y) (fp32), 2e-2 * RMS(y) (bf16)
and 5e-2 * RMS(y) (MXFP4, oracle on the same dequantised bits)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_router_amd as moe
import synthetic
from gpu_helpers import DeviceLayer, check_stages, compare, desc_of, run, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def small_case(name, **kw):
    base = dict(T=77, d=1024, L=512, F=512, n=32, k=4)
    base.update(kw)
    return synthetic.small(name=name, **base)


def run_and_compare(p, tokens=None, route_tokens=None, layer=None):
    say("case %s T=%d d=%d L=%d F=%d n=%d k=%d weights=%s in_norm=%s" % (p.name, p.T, p.d, p.L, p.F, p.n, p.k,
                                                                      p.weights, p.in_norm))
    layer = layer or DeviceLayer(p)
    x = synthetic.inputs(p)
    gpu = run(layer, x)
    res = compare(p, layer.host, x, gpu, tokens=tokens, route_tokens=route_tokens, label=p.name)
    if p.act == "bf16":
        check_stages(p, layer.host, x, gpu, np.arange(p.T) if tokens is None else tokens, label=p.name)
    return res, gpu


def test_c0_tiny_fp32_layer():
    p = synthetic.PRESETS["c0"]
    run_and_compare(p)


def test_c0_relu_vs_swiglu_fp32():
    p = synthetic.Preset(**dict(synthetic.PRESETS["c0"].cfg(), name="c0_swiglu", kind="swiglu3", T=33))
    run_and_compare(p)


@pytest.mark.parametrize("weights", ["bf16", "mxfp4"])
@pytest.mark.parametrize("in_norm", ["none", "centered", "input_scaled"])
def test_small_decode_shape(weights, in_norm):
    # ~10 tokens per expert: every expert on the streaming kernel
    run_and_compare(small_case("small_decode_%s_%s" % (weights, in_norm), weights=weights, in_norm=in_norm))


def test_mxfp4_streaming_scale_chunks():
    # MXFP4 streaming items hold the scale words of up to 16 of a wave's 128-wide K groups at a time: the
    # down-projection (K = 8704: 17 groups per wave) and GEMM1 (K = 8704) run a chunk of 16 groups and a
    # ragged chunk of one; GEMM2 (K = 512) has one group per wave
    run_and_compare(small_case("mxfp4_scale_chunks", T=24, d=8704, L=8704, F=512, n=16, k=2, weights="mxfp4"))


@pytest.mark.parametrize("weights", ["bf16", "mxfp4"])
def test_small_prefill_shape(weights):
    # ~300 tokens per expert: tiled kernels for the dense and grouped GEMMs
    p = small_case("small_prefill_" + weights, T=1203, n=16, k=4, weights=weights)
    tok = synthetic.sample_tokens(p.T, 160, seed=5)
    run_and_compare(p, tokens=tok)


@pytest.mark.parametrize("T,res_gate", [(32, "linear"), (77, "linear"), (128, "linear"), (100, "none")])
def test_up_projection_k_sliced(T, res_gate):
    # 32..128 rows: the up-projection on half-height tiles whose 4 K slices of 512 store fp32 planes
    # that a second kernel adds in slice order before the residual (or plain) epilogue
    p = small_case("up_split_T%d_%s" % (T, res_gate), T=T, d=2048, L=2048, F=512, n=32, k=4,
                   res_gate=res_gate)
    layer = DeviceLayer(p)
    _, gpu = run_and_compare(p, layer=layer)
    if T == 77:
        # the fp16 weight format through the same slices: bitwise the bf16 format's results
        got = run(f16_weight_layer(layer), synthetic.inputs(p))
        for key in gpu:
            np.testing.assert_array_equal(got[key], gpu[key], err_msg=key)


def test_small_skewed_mixed_tiles():
    # a Zipf selection bias: hot experts on the tiled kernel, cold ones streamed, some empty
    p = small_case("small_skew", T=700, n=32, k=4, router_bias="zipf")
    res, gpu = run_and_compare(p, tokens=synthetic.sample_tokens(p.T, 160, seed=6))
    counts = gpu["expert_counts"]
    assert counts.max() > 32 and (counts <= 32).any()


def test_stream_items_pipelined_across_tiles():
    # ~19 tokens per expert over 256 experts: every expert streamed as a full 16-row tile plus a short
    # one, and more items than the streaming grid, so each workgroup runs several items back to back
    # (the next item's first loads go out under the previous item's epilogue) over tiles of both sizes
    p = small_case("stream_pipelined", T=600, n=256, k=8)
    res, gpu = run_and_compare(p, tokens=synthetic.sample_tokens(p.T, 200, seed=9))
    counts = gpu["expert_counts"]
    # (an average of <= 32 rows per expert streams every expert, whatever its count)
    assert -(-p.T * p.k // p.n) <= 32
    assert (counts > 16).sum() > 100 and ((counts % 16) <= 8).sum() > 50


def test_batch_rows_past_2gib():
    # T * k * d_ff * 2 bytes of expert activations exceed 2 GiB: the tile kernels address GEMM2's rows from
    # each tile's first row (32-bit lane offsets), so slots whose rows sit past 2 GiB of that buffer are
    # computed like the first ones; checked on tokens with such slots, and a few others
    p = small_case("rows_past_2gib", T=131072, d=512, L=512, F=2048, n=16, k=8)
    assert p.T * p.k * p.F * 2 > 2 ** 31
    layer = DeviceLayer(p)
    x = synthetic.inputs(p)
    gpu = run(layer, x, stages=False)
    far = np.flatnonzero((gpu["pos"].astype(np.int64) * p.F * 2 >= 2 ** 31).any(axis=1))
    assert far.size > 1000
    rng = np.random.default_rng(7)
    tok = np.unique(np.concatenate([rng.choice(far, 12, replace=False), rng.choice(p.T, 4, replace=False),
                                    [0, p.T - 1]]))
    compare(p, layer.host, x, gpu, tokens=tok, route_tokens=synthetic.sample_tokens(p.T, 2048, seed=8))


def test_single_token_and_top1():
    run_and_compare(small_case("t1", T=1))
    run_and_compare(small_case("top1", T=50, k=1))


@pytest.mark.parametrize("T", [1, 16, 128])
def test_mxfp4_batch_edges(T):
    # MXFP4 dense projections take 16-row items of four weight blocks up to T = 128 (one row, one full tile,
    # eight tiles); grouped items of four blocks on every expert
    run_and_compare(small_case("mxfp4_T%d" % T, T=T, weights="mxfp4"))


def test_mxfp4_k_equals_n():
    run_and_compare(small_case("mxfp4_k_eq_n", T=40, n=16, k=16, weights="mxfp4"))


def test_k_equals_n():
    run_and_compare(small_case("k_eq_n", T=40, n=16, k=16))


def test_zero_rows_tie_to_lowest_ids():
    p = small_case("zeros", T=20)
    layer = DeviceLayer(p)
    x = synthetic.inputs(p)
    x[3] = 0
    x[11] = 0
    gpu = run(layer, x)
    for r in (3, 11):
        assert list(gpu["topk_idx"][r]) == list(range(p.k))
        np.testing.assert_allclose(gpu["topk_w"][r], 1.0 / p.k, rtol=1e-6)
    # zero rows are excluded from the graded routing (margin 0) but their outputs still match
    compare(p, layer.host, x, gpu, label="zeros")
    check_stages(p, layer.host, x, gpu, np.arange(p.T), label="zeros")


def test_empty_batch_enqueues_nothing():
    p = small_case("empty", T=0)
    layer = DeviceLayer(p)
    out = torch.empty((0, p.d), dtype=torch.float32, device="cuda")
    x = torch.empty((0, p.d), dtype=torch.int16, device="cuda")
    dv = layer.dev
    moe.moe_layer_forward(desc_of(p, 0), x, dv["router_w"], dv["down_w"], dv["w1"], dv["w2"], dv["up_w"],
                          layer.gains(), out)
    torch.cuda.synchronize()


def test_deterministic_and_reused_workspace():
    p = small_case("det", T=300, n=16, k=4)
    layer = DeviceLayer(p)
    x = synthetic.inputs(p)
    ws = torch.full((moe.moe_workspace_bytes(desc_of(p, p.T)),), 0x5A, dtype=torch.uint8, device="cuda")
    a = run(layer, x, workspace=ws)
    b = run(layer, x, workspace=ws)
    for k_ in a:
        np.testing.assert_array_equal(a[k_], b[k_], err_msg=k_)
    # rows are independent: with the same kernels (every expert streamed at
    # these batch sizes) a prefix batch gives the same rows bit for bit
    d = run(layer, x[:60])
    c = run(layer, x[:23])
    np.testing.assert_array_equal(c["out"], d["out"][:23])
    np.testing.assert_array_equal(c["topk_idx"], d["topk_idx"][:23])


def test_router_topk_stage_entry_point():
    p = small_case("router_stage", T=130, n=32, k=4, router_bias="zipf")
    prm = synthetic.layer_params(p)
    x = synthetic.inputs(p)
    idx = torch.empty((p.T, p.k), dtype=torch.int32, device="cuda")
    w = torch.empty((p.T, p.k), dtype=torch.float32, device="cuda")
    lg = torch.empty((p.T, p.n), dtype=torch.float32, device="cuda")
    moe.moe_router_topk(desc_of(p), to_dev(x), to_dev(prm["router_w"]), to_dev(prm["bias"]), idx, w, logits=lg)
    torch.cuda.synchronize()
    r = oracle.forward(p.cfg(), dict(prm, x=x), want_outputs=False)
    np.testing.assert_allclose(lg.cpu().numpy(), r["logits"], rtol=0, atol=1e-4)
    gpu = {"topk_idx": idx.cpu().numpy(), "topk_w": w.cpu().numpy()}
    from gpu_helpers import check_routing
    check_routing(p, prm, x, gpu, np.arange(p.T), "router_stage")


def test_router_topk_k_sliced():
    # n = 256 and T > 128: the router GEMM runs on the tiled kernel with K in
    # 8 slices of 512, whose partial planes the selection adds in order; the
    # same call without a workspace runs unsliced into the given logits
    p = small_case("router_sliced", T=600, d=4096, n=256, k=8, router_bias="zipf")
    prm = {"router_w": synthetic.normal_bf16(p.layer_seed, "router_w", p.n * p.d, p.w_std).reshape(p.n, p.d),
           "bias": synthetic.zipf_bias(p.n)}
    x = synthetic.inputs(p)
    desc = desc_of(p)
    ws = torch.empty(moe.moe_router_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    assert ws.numel() >= 8 * p.T * p.n * 4
    r = oracle.forward(p.cfg(), dict(prm, x=x), want_outputs=False)
    from gpu_helpers import check_routing
    for label, workspace in (("sliced", ws), ("unsliced", None)):
        idx = torch.empty((p.T, p.k), dtype=torch.int32, device="cuda")
        w = torch.empty((p.T, p.k), dtype=torch.float32, device="cuda")
        lg = torch.full((p.T, p.n), float("nan"), dtype=torch.float32, device="cuda")
        moe.moe_router_topk(desc, to_dev(x), to_dev(prm["router_w"]), to_dev(prm["bias"]), idx, w, logits=lg,
                            workspace=workspace)
        torch.cuda.synchronize()
        np.testing.assert_allclose(lg.cpu().numpy(), r["logits"], rtol=0, atol=1e-4, err_msg=label)
        check_routing(p, prm, x, {"topk_idx": idx.cpu().numpy(), "topk_w": w.cpu().numpy()}, np.arange(p.T),
                      "router " + label)


@pytest.mark.parametrize("T,k,n", [(1, 1, 1), (5, 2, 8), (1000, 8, 256), (3000, 4, 16), (2500, 8, 256)])
def test_permute_stage_entry_point(T, k, n):
    rng = np.random.default_rng(T * 7 + n)
    if n > 1:
        # skewed: low ids far more likely
        pr = 1.0 / np.arange(1, n + 1) ** 1.2
        pr /= pr.sum()
        idx = np.stack([rng.choice(n, size=k, replace=False, p=pr) for _ in range(T)]).astype(np.int32)
    else:
        idx = np.zeros((T, k), np.int32)
    dev = {nm: torch.empty(sz, dtype=torch.int32, device="cuda") for nm, sz in
           (("counts", n), ("offsets", n + 1), ("perm_tok", T * k), ("perm_slot", T * k), ("pos", T * k))}
    moe.moe_permute(T, k, n, to_dev(idx), dev["counts"], dev["offsets"], dev["perm_tok"], dev["perm_slot"],
                    dev["pos"])
    torch.cuda.synchronize()
    ref = oracle.permute(idx, n)
    for nm in dev:
        np.testing.assert_array_equal(dev[nm].cpu().numpy().reshape(-1), ref[nm].reshape(-1), err_msg=nm)


@pytest.mark.parametrize("T,n", [(77, 32), (1203, 16)])
def test_bf16_intermediates(T, n):
    # interm_dtype = bf16: z, SwiGLU output and m kept in bf16 (the range-safe option)
    p = small_case("bf16_interm_T%d" % T, T=T, n=n, interm="bf16")
    run_and_compare(p, tokens=synthetic.sample_tokens(p.T, 120, seed=7))


def test_fp16_range_overflow_is_loud():
    # a z value beyond the fp16 range becomes inf and poisons its token's outputs (never silently clipped)
    p = small_case("f16_overflow", T=8)
    layer = DeviceLayer(p)
    x = synthetic.inputs(p)
    big = synthetic.bf16_to_f32(x[5]) * 3.0e5
    x[5] = synthetic.f32_to_bf16(big)
    gpu = run(layer, x, stages=False)
    assert not np.isfinite(gpu["out"][5]).all()
    assert np.isfinite(gpu["out"][[0, 1, 2, 3, 4, 6, 7]]).all()


def test_bf16_to_f16_conversion_every_pattern():
    # every bf16 bit pattern against numpy's round-to-nearest-even float16 cast
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(over="ignore"):
        ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float16).view(np.uint16)
    src = to_dev(bits)
    dst = torch.empty_like(src)
    moe.moe_convert_bf16_to_f16(src, dst, bits.size)
    moe.moe_convert_bf16_to_f16(src, src, bits.size)  # in place
    torch.cuda.synchronize()
    nan = np.isnan(ref.view(np.float16))
    for got in (dst.cpu().numpy().view(np.uint16), src.cpu().numpy().view(np.uint16)):
        np.testing.assert_array_equal(got[~nan], ref[~nan])
        assert np.isnan(got[nan].view(np.float16)).all()


def f16_weight_layer(layer: DeviceLayer) -> DeviceLayer:
    """The same layer with expert_w1, expert_w2 and up_w converted on the
    device to the fp16 weight format (down_w stays bf16)."""
    lay = DeviceLayer.__new__(DeviceLayer)
    lay.p = dataclasses.replace(layer.p, name=layer.p.name + "_f16w", weights="f16")
    lay.host, lay.dev = layer.host, dict(layer.dev)
    for key in ("w1", "w2", "up_w"):
        t = layer.dev[key]
        c = torch.empty_like(t)
        moe.moe_convert_bf16_to_f16(t, c, t.numel())
        lay.dev[key] = c
    return lay


@pytest.mark.parametrize("T,n", [(77, 32), (1203, 16)])
def test_f16_weight_format(T, n):
    # fp16-stored weights feed the fp16 GEMMs the bits the bf16 format converts
    # to as it reads them: every output and intermediate is bitwise the same,
    # and both meet the oracle's bar on the checkpoint's bf16 weights
    p = small_case("f16w_T%d" % T, T=T, n=n)
    layer = DeviceLayer(p)
    x = synthetic.inputs(p)
    ref = run(layer, x)
    got = run(f16_weight_layer(layer), x)
    for key in ref:
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    compare(p, layer.host, x, got, tokens=synthetic.sample_tokens(p.T, 120, seed=9), label=p.name + " f16 weights")
