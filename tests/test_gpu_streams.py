"""Streams and capture: the Python conveniences allocate their outputs and workspace on the
stream the kernels run on, and a process's very first prefill may be made inside a HIP-graph
capture (the library's one lazily filled value, a per-device occupancy count, is then taken
during the capture).

Both compare against the same call made eagerly on the default stream, bit for bit."""
import os
import subprocess
import sys
import textwrap

import pytest
import torch

from linear_recurrent_attention_gated_amd import gdn
from linear_recurrent_attention_gated_amd.inputs import make_inputs
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_prefill_and_decode_on_a_side_stream_equal_default_stream():
    d = {k: v.cuda() for k, v in make_inputs(1, 700, 2, 4, 128, 128, seed=51,
                                             state_std=0.1).items()}
    say("side stream prefill")
    o_ref, s_ref = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], chunk=64)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for r in range(3):
        o, s = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], chunk=64,
                           stream=side)
        # allocation churn on the current stream while the side stream's kernels run: a
        # workspace freed by the call above must not be handed to this work
        junk = [torch.full((1 << 22,), float(r + i), device="cuda") for i in range(8)]
        outs.append((o, s, junk))
    side.synchronize()
    torch.cuda.synchronize()
    for o, s, _ in outs:
        assert torch.equal(o, o_ref) and torch.equal(s, s_ref)

    say("side stream decode")
    q, k, v = (d[x][:, 0].contiguous() for x in ("q", "k", "v"))
    g, b = d["g"][:, 0].contiguous(), d["beta"][:, 0].contiguous()
    st_ref, st = d["state"].clone(), d["state"].clone()
    od_ref = gdn.decode_step(q, k, v, g, b, st_ref)
    torch.cuda.synchronize()
    side.wait_stream(torch.cuda.current_stream())
    od = gdn.decode_step(q, k, v, g, b, st, stream=side)
    side.synchronize()
    assert torch.equal(od, od_ref) and torch.equal(st, st_ref)


CAPTURE_FIRST = textwrap.dedent("""
    import sys, torch
    sys.path.insert(0, {root!r})
    from linear_recurrent_attention_gated_amd import gdn
    from linear_recurrent_attention_gated_amd.inputs import make_inputs
    d = {{k: v.cuda() for k, v in make_inputs(1, 300, 2, 4, 64, 128, seed=52, state_std=0.1).items()}}
    nb = gdn.gdn_prefill_workspace_bytes(1, 300, 2, 4, 64, 128, 32, torch.bfloat16)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    o, s = torch.empty_like(d["v"]), torch.empty_like(d["state"])
    torch.cuda.synchronize()
    print("capture: first prefill of this process", flush=True)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdn.gdn_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], o, s, 32, ws)
    torch.cuda.synchronize()
    o_e, s_e = torch.empty_like(o), torch.empty_like(s)
    for r in range(3):
        graph.replay()
        gdn.gdn_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], o_e, s_e, 32, ws)
        torch.cuda.synchronize()
        assert torch.equal(o, o_e) and torch.equal(s, s_e), r
        print("replay", r, "equals eager", flush=True)
""")


def test_first_prefill_of_a_process_inside_graph_capture():
    say("capture-first prefill in a child process")
    r = subprocess.run([sys.executable, "-c", CAPTURE_FIRST.format(root=ROOT)],
                       capture_output=True, text=True, timeout=110)
    print(r.stdout, r.stderr[-2000:], flush=True)
    assert r.returncode == 0
