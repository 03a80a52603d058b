"""MXFP8 activations at the two expert GEMMs (act_quant = MXFP8) with MXFP4
weights, through the C ABI.

Reading of the tolerance: the quantized activations are part of what the
layer computes in this mode, as the MXFP4 weights are.  The oracle applies
the same OCP MX quantizer (E4M3 elements, one power-of-two scale per 32
along K) to the stored latent z and SwiGLU output and evaluates everything
else in fp64; the device's outputs must match it to 5e-2 * RMS(y), the MXFP4
bar.  A token whose quantized latent differs from the oracle's (one E4M3
code flipped where the device's and the oracle's stored z sit on either side
of a rounding midpoint) is evaluated by the oracle on the device's quantized
latent, as a near-tie token is on the device's experts: one flipped code
moves the SwiGLU output enough to flip a few percent of its codes in turn.
The stage checks are bit-exact on the quantized codes and scales (the
oracle's quantizer applied to the device's own stored values) and graded to
one ulp on the GEMM outputs that read them.  How far the mode moves the
layer from the unquantized oracle is reported, not graded."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_router_amd as moe
import synthetic
from gpu_helpers import DeviceLayer, check_stages, compare, run, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def q8_case(name, **kw):
    base = dict(T=77, d=1024, L=512, F=512, n=32, k=4, weights="mxfp4", act_quant="mxfp8")
    base.update(kw)
    return synthetic.small(name=name, **base)


def run_q8(p, tokens=None):
    layer = DeviceLayer(p)
    x = synthetic.inputs(p)
    gpu = run(layer, x)
    check_stages(p, layer.host, x, gpu, np.arange(p.T), label=p.name)
    res = compare(p, layer.host, x, gpu, tokens=tokens, label=p.name)
    # what the quantization costs, against the oracle without it (reported only)
    tok = np.arange(p.T) if tokens is None else tokens
    r0 = oracle.forward(dict(p.cfg(), act_quant="none"), dict(layer.host, x=x), tokens=tok)
    rms = float(np.sqrt(np.mean(r0["y"] ** 2)))
    say("%s: max|dout| against the unquantized oracle %.3g * RMS(y)" % (
        p.name, float(np.abs(gpu["out"][tok] - r0["out"]).max()) / rms))
    return res, gpu


@pytest.mark.parametrize("in_norm", ["none", "centered"])
def test_q8_streamed_experts(in_norm):
    # ~10 tokens per expert: every expert on the streaming kernel (operands decoded to bf16)
    run_q8(q8_case("q8_stream_" + in_norm, in_norm=in_norm))


def test_q8_tiled_experts():
    # ~300 tokens per expert: full, half and tall tiles on the scaled fp8 x fp4 MFMA
    p = q8_case("q8_tiles", T=1203, n=16, k=4)
    _, gpu = run_q8(p, tokens=synthetic.sample_tokens(p.T, 160, seed=5))
    c = gpu["expert_counts"]
    say("q8_tiles tokens/expert: %s" % sorted(c.tolist()))
    assert c.min() > 128


def test_q8_mixed_tiles_skewed():
    # a Zipf selection bias: hot experts tiled, cold ones streamed, some empty; a ragged tile height
    p = q8_case("q8_skew", T=700, n=32, k=4, router_bias="zipf")
    _, gpu = run_q8(p, tokens=synthetic.sample_tokens(p.T, 160, seed=6))
    c = gpu["expert_counts"]
    assert c.max() > 32 and (c <= 32).any()


def test_q8_bf16_intermediates():
    # z and the SwiGLU output stored as bf16 before quantization
    run_q8(q8_case("q8_bf16_interm", T=300, n=16, k=4, interm="bf16"),
           tokens=synthetic.sample_tokens(300, 100, seed=7))
