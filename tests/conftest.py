import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def read_golden(name):
    """Parse a golden fixture: 'key v1 v2 ...' lines, '#' comments."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            out[parts[0]] = [float(v) for v in parts[1:]]
    return out


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def preset_desc(p, T=None):
    """The moe_desc of a synthetic preset (T: rows of one call, default the
    preset's chunk)."""
    import sparse_mixture_experts_router_amd as moe
    return moe.make_desc(p.chunk_T if T is None else T, p.d, p.L, p.n, p.k, p.F, expert_kind=p.kind, act=p.act,
                         router=p.router_w, weights=p.weights, in_norm=p.in_norm, expert_norm=p.expert_norm,
                         res_gate=p.res_gate, bias_in_weights=p.bias_in_weights, eps_in=p.eps_in,
                         eps_expert=p.eps_expert, interm=p.interm, router_fn=p.router_fn, out_mult=p.out_mult,
                         routed_scale=p.routed_scale, latent_norm=p.latent_norm, eps_latent=p.eps_latent,
                         out_norm=p.out_norm, eps_out=p.eps_out, res_tau=p.res_tau, res_floor=p.res_floor,
                         act_quant=p.act_quant)
