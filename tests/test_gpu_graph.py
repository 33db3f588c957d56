"""HIP-graph capture of the library's launches: a 30-layer decode token (30 back-to-back
gdn_decode_step calls, each layer's state updated in place) and a blockwise prefill,
captured once and replayed several times.  Every replay is checked against the same
calls made eagerly on a copy of the buffers, with the program's own eager work and
synchronisations between replays; the first decode replay is also checked against the
fp64 oracle.  The library enqueues kernels only (no memset or allocation), so the
captured graph holds kernel nodes only."""
import numpy as np
import pytest
import torch

from linear_recurrent_attention_gated_amd import gdn
from linear_recurrent_attention_gated_amd.inputs import decode_inputs, make_inputs
from oracle import gdn_oracle as orc
from tests.gpu_util import TOL_O, TOL_S, nrel, np32, say

pytestmark = pytest.mark.gpu

LAYERS = 30
REPLAYS = 4


def _eager_noise(i):
    # unrelated eager work between replays (reductions over many blocks, a copy)
    x = torch.randn(1 << 20, device="cuda", generator=torch.Generator("cuda").manual_seed(i))
    return float(x.abs().sum().item() + x.clone().max().item())


def test_decode_30_layers_graph_replays_match_eager():
    host = [decode_inputs(l) for l in range(LAYERS)]
    dev = [{k: v.cuda() for k, v in d.items()} for d in host]
    st_g = [d["state"].clone() for d in dev]
    st_e = [d["state"].clone() for d in dev]
    o_g = [torch.empty_like(d["v"]) for d in dev]
    o_e = [torch.empty_like(d["v"]) for d in dev]

    def step(states, outs):
        for l, d in enumerate(dev):
            gdn.gdn_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], states[l], states[l],
                                outs[l])

    say("graph capture: decode", LAYERS, "layers")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(st_g, o_g)
    torch.cuda.synchronize()
    # capture enqueues nothing: the states are untouched until the first replay
    for l in range(LAYERS):
        assert torch.equal(st_g[l], dev[l]["state"])

    for r in range(REPLAYS):
        say("decode replay", r)
        graph.replay()
        step(st_e, o_e)
        torch.cuda.synchronize()
        _eager_noise(r)
        for l in range(LAYERS):
            assert torch.equal(o_g[l], o_e[l]), (r, l)
            assert torch.equal(st_g[l], st_e[l]), (r, l)
        if r == 0:
            for l in (0, 17, 29):
                d = {k: v.float().numpy() for k, v in host[l].items()}
                o_ref, s_ref = orc.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                               d["state"].astype(np.float64))
                assert nrel(np32(o_g[l]), o_ref) < TOL_O
                assert nrel(st_g[l].cpu().numpy(), s_ref) < 1e-6


def test_prefill_graph_replays_match_eager():
    B, T, Hk, Hv, dk, dv, chunk = 1, 300, 2, 4, 128, 128, 64
    d = {k: (None if v is None else v.cuda())
         for k, v in make_inputs(B, T, Hk, Hv, dk, dv, seed=41, state_std=0.3).items()}
    nb = gdn.gdn_prefill_workspace_bytes(B, T, Hk, Hv, dk, dv, chunk, torch.bfloat16)
    ws_g = torch.empty(nb, dtype=torch.uint8, device="cuda")
    ws_e = torch.empty_like(ws_g)
    o_g, o_e = torch.empty_like(d["v"]), torch.empty_like(d["v"])
    s_g, s_e = torch.empty_like(d["state"]), torch.empty_like(d["state"])
    # one state buffer chained through the replays: state_in = state_out of the last call
    s_g.copy_(d["state"])
    s_e.copy_(d["state"])

    say("graph capture: prefill", (B, T, Hk, Hv, dk, dv, chunk))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdn.gdn_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], s_g, o_g, s_g, chunk, ws_g)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        say("prefill replay", r)
        graph.replay()
        gdn.gdn_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], s_e, o_e, s_e, chunk, ws_e)
        torch.cuda.synchronize()
        _eager_noise(100 + r)
        assert torch.equal(o_g, o_e), r
        assert torch.equal(s_g, s_e), r
    assert torch.all(torch.isfinite(s_g))
