"""A layer forward captured in a HIP graph (torch.cuda.CUDAGraph) replays to
the eager forward's bits.  Every kernel of the forward launches on the
caller's stream, and the forward allocates nothing and clears no memory
with a memset (its counters are cleared by its own kernels), so the graph
holds kernel nodes only.  Replays alternate with eager calls on another
input; every replay and every eager call is checked bit for bit against
the eager result of its input."""
import dataclasses

import pytest
import torch

import sparse_mixture_experts_router_amd as moe
import synthetic
from gpu_helpers import DeviceLayer, desc_of, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


CASES = {
    # ~10 tokens per expert: streaming kernels, the K-sliced router
    "decode": dict(T=77, d=1024, L=512, F=512, n=32, k=4),
    # ~300 tokens per expert: tiled kernels
    "prefill": dict(T=1203, d=1024, L=512, F=512, n=16, k=4),
}


@pytest.mark.parametrize("case", ["decode", "prefill", "muse", "f16"])
def test_graph_replays_match_eager(case):
    if case == "muse":
        p = synthetic.muse("graph_muse", **dict(CASES["decode"], layer_seed=11, input_seed=12))
    else:
        p = synthetic.small(name="graph_" + case, **CASES["prefill" if case == "prefill" else "decode"])
    say("graph case %s T=%d n=%d" % (case, p.T, p.n))
    layer = DeviceLayer(p)
    dv = dict(layer.dev)
    desc = desc_of(p)
    if case == "f16":
        for key in ("w1", "w2", "up_w"):
            c = torch.empty_like(dv[key])
            moe.moe_convert_bf16_to_f16(dv[key], c, c.numel())
            dv[key] = c
        desc = desc_of(dataclasses.replace(p, weights="f16"))
    xs = [to_dev(synthetic.inputs(p)), to_dev(synthetic.inputs(dataclasses.replace(p, input_seed=p.input_seed + 1)))]
    xin = torch.empty_like(xs[0])
    out = torch.empty((p.T, p.d), dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    gains = layer.gains()

    def fwd(stream):
        moe.moe_layer_forward(desc, xin, dv["router_w"], dv["down_w"], dv["w1"], dv["w2"], dv["up_w"], gains, out,
                              workspace=ws, stream=stream)

    refs = []
    for x in xs:
        xin.copy_(x)
        fwd(torch.cuda.current_stream())
        torch.cuda.synchronize()
        refs.append(out.clone())
    assert not torch.equal(refs[0], refs[1])

    # capture on a side stream (torch's recipe: one warm-up call there first)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd(torch.cuda.current_stream())
    torch.cuda.synchronize()

    for rep in range(6):
        i = rep % 2
        xin.copy_(xs[i])
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, refs[i]), "replay %d" % rep
        xin.copy_(xs[1 - i])
        fwd(torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert torch.equal(out, refs[1 - i]), "eager call after replay %d" % rep
