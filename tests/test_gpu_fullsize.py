"""GPU parity at the 816B-A42B layer's real shape (d=8192, L=F=4096, n=256,
k=8), in the launch configuration the benchmark times: routing checked on
every token (against the oracle's own routing, and stage by stage: logits,
experts and weights against the oracle on the device's own branch input and
logits), the permutation bit-exact on every token, and layer outputs on
OUT_SAMPLE seeded tokens the oracle evaluates one by one (rows are
independent)."""
import dataclasses

import numpy as np
import pytest
import torch

import sparse_mixture_experts_router_amd as moe

import synthetic
from gpu_helpers import DeviceLayer, check_stages, compare, run, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def layer_host():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    say("generating the seed-1 layer (bf16 and MXFP4 forms)")
    return synthetic.layer_params(synthetic.PRESETS["c1"], formats=("bf16", "mxfp4"))


@pytest.fixture(scope="module")
def bf16_layer(layer_host):
    say("uploading bf16 layer")
    return DeviceLayer(synthetic.PRESETS["c1"], host={k: v for k, v in layer_host.items() if "@" not in k})


BIG = ("router_w", "down_w", "w1", "w2", "up_w")
OUT_SAMPLE = 256


def cold_tokens(gpu, small_max: int = 32, count: int = 8) -> np.ndarray:
    """Tokens with at least one expert of at most small_max tokens (the
    experts the streaming kernel runs at large batches), up to `count`."""
    cold = gpu["expert_counts"] <= small_max
    hit = np.flatnonzero(cold[gpu["topk_idx"]].any(axis=1))
    return hit[:count].astype(np.int64)


def preset_layer(p, layer_host, base: DeviceLayer):
    """A DeviceLayer for preset p sharing the seed-1 device weights of `base`
    (MXFP4 presets get the MXFP4 forms of the same draws), with p's own small
    parameter vectors (gains, gate, bias)."""
    host = {k: layer_host[k] for k in BIG}
    lay = DeviceLayer.__new__(DeviceLayer)
    lay.p, lay.host, lay.dev = p, host, {k: base.dev[k] for k in BIG}
    if p.weights == "mxfp4":
        for k in ("down_w", "w1", "w2", "up_w"):
            host[k] = layer_host[k + "@mxfp4"]
            lay.dev[k] = to_dev(host[k])
    for k, v in synthetic.gains(p).items():
        host[k] = v
        lay.dev[k] = to_dev(v)
    return lay


def test_c1_decode_T64(bf16_layer):
    p = synthetic.PRESETS["c1"]
    x = synthetic.inputs(p)
    gpu = run(bf16_layer, x)
    touched = int((gpu["expert_counts"] > 0).sum())
    say("c1 touched experts: %d" % touched)
    compare(p, bf16_layer.host, x, gpu, label="c1")
    check_stages(p, bf16_layer.host, x, gpu, synthetic.sample_tokens(p.T, 4, seed=11), label="c1")


def test_c2_prefill_T8192(layer_host, bf16_layer):
    p = synthetic.PRESETS["c2"]
    x = synthetic.inputs(p)
    gpu = run(bf16_layer, x)
    c = gpu["expert_counts"]
    say("c2 tokens/expert min %d max %d" % (c.min(), c.max()))
    compare(p, bf16_layer.host, x, gpu, tokens=synthetic.sample_tokens(p.T, OUT_SAMPLE, seed=21), label="c2")
    check_stages(p, bf16_layer.host, x, gpu, synthetic.sample_tokens(p.T, 4, seed=23), label="c2")


def test_c3_skewed_T16384(layer_host, bf16_layer):
    p = synthetic.PRESETS["c3"]
    lay = preset_layer(p, layer_host, bf16_layer)
    x = synthetic.inputs(p)
    gpu = run(lay, x)
    c = gpu["expert_counts"]
    say("c3 hottest expert %d tokens (%.1f%% of tokens), empty experts %d, experts with <=5 tokens %d" % (
        c.max(), 100.0 * c.max() / p.T, int((c == 0).sum()), int((c <= 5).sum())))
    assert (c == 0).any() and c.max() > 0.5 * p.T
    # the output sample holds tokens routed to cold experts (the streamed ones), as well as random ones
    cold = cold_tokens(gpu)
    assert cold.size > 0, "no token reached an expert of <= 32 tokens"
    tok = np.unique(np.concatenate([synthetic.sample_tokens(p.T, OUT_SAMPLE, seed=31), cold]))
    compare(p, lay.host, x, gpu, tokens=tok, label="c3")
    check_stages(p, lay.host, x, gpu, np.unique(np.concatenate([tok[:3], cold[:2]])), label="c3")


def test_c1m_mxfp4_decode_T64(layer_host, bf16_layer):
    # the decode batch on the MXFP4 weights (streaming kernel, codes dequantised in registers): every
    # token's outputs against the oracle on the same dequantised bits
    p = synthetic.PRESETS["c1m"]
    lay = preset_layer(p, layer_host, bf16_layer)
    x = synthetic.inputs(p)
    gpu = run(lay, x)
    compare(p, lay.host, x, gpu, label="c1m")
    check_stages(p, lay.host, x, gpu, np.arange(4), label="c1m")


@pytest.mark.parametrize("name", ["c4c", "c4i"])
@pytest.mark.parametrize("which", ["first", "last"])
def test_c4_mxfp4_chunks(name, which, layer_host, bf16_layer):
    p = synthetic.PRESETS[name]
    lay = preset_layer(p, layer_host, bf16_layer)
    chunk = 0 if which == "first" else p.chunks - 1
    x = synthetic.inputs(p, chunk=chunk)
    gpu = run(lay, x)
    compare(p, lay.host, x, gpu, tokens=synthetic.sample_tokens(p.chunk_T, OUT_SAMPLE, seed=40 + chunk),
            label="%s chunk %d" % (name, chunk))
    check_stages(p, lay.host, x, gpu, synthetic.sample_tokens(p.chunk_T, 3, seed=60 + chunk),
                 label="%s chunk %d" % (name, chunk))


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_f16_weight_format_full_size(name, bf16_layer):
    # the fp16 weight format at the real shape: bitwise the bf16 format's results
    p = synthetic.PRESETS[name]
    x = synthetic.inputs(p)
    ref = run(bf16_layer, x)
    lay = DeviceLayer.__new__(DeviceLayer)
    lay.p = dataclasses.replace(p, weights="f16")
    lay.host, lay.dev = bf16_layer.host, dict(bf16_layer.dev)
    for key in ("w1", "w2", "up_w"):
        t = bf16_layer.dev[key]
        c = torch.empty_like(t)
        moe.moe_convert_bf16_to_f16(t, c, t.numel())
        lay.dev[key] = c
    got = run(lay, x)
    del lay
    torch.cuda.empty_cache()
    for key in ref:
        np.testing.assert_array_equal(got[key], ref[key], err_msg="%s %s" % (name, key))


@pytest.mark.parametrize("name", ["m1", "m2"])
def test_muse_sublayer_full_size(name, layer_host, bf16_layer):
    # sigmoid router with a correction bias, latent pre-norm, input-scaled
    # output norm and the alpha/beta residual gate around the same layer
    p = synthetic.PRESETS[name]
    lay = preset_layer(p, layer_host, bf16_layer)
    x = synthetic.inputs(p)
    gpu = run(lay, x)
    w = gpu["topk_w"]
    say("%s weight sums: min %.6f max %.6f" % (name, w.sum(1).min(), w.sum(1).max()))
    np.testing.assert_allclose(w.sum(1), p.routed_scale, rtol=1e-5)
    if p.T <= 64:
        compare(p, lay.host, x, gpu, label=name)
        st = synthetic.sample_tokens(p.T, 4, seed=71)
    else:
        compare(p, lay.host, x, gpu, tokens=synthetic.sample_tokens(p.T, OUT_SAMPLE, seed=72), label=name)
        st = synthetic.sample_tokens(p.T, 4, seed=74)
    check_stages(p, lay.host, x, gpu, st, label=name)


def test_c4q_mxfp8_activations(layer_host, bf16_layer):
    # the c4 workload's first chunk with MXFP8 activations at the expert GEMMs (the scaled fp8 x fp4 MFMA
    # on the tiled experts), graded against the oracle with the same quantizer (MXFP4 bar)
    p = synthetic.PRESETS["c4q"]
    lay = preset_layer(p, layer_host, bf16_layer)
    x = synthetic.inputs(p, chunk=0)
    gpu = run(lay, x)
    tok = synthetic.sample_tokens(p.chunk_T, OUT_SAMPLE, seed=80)
    check_stages(p, lay.host, x, gpu, tok[:3], label="c4q chunk 0")
    compare(p, lay.host, x, gpu, tokens=tok, label="c4q chunk 0")
    import oracle
    t = dict(lay.host, x=x)
    r0 = oracle.forward(dict(p.cfg(), act_quant="none"), t, tokens=tok[:64])
    rms = float(np.sqrt(np.mean(r0["y"] ** 2)))
    say("c4q: max|dout| against the unquantized oracle %.3g * RMS(y) (reported)" % (
        float(np.abs(gpu["out"][tok[:64]] - r0["out"]).max()) / rms))
