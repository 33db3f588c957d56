"""gdn_prefill_noalloc (the library's fixed device array as the workspace) against gdn_prefill
with a caller-allocated one-pass workspace, through the C ABI: two calls in a row, the second
with a smaller input, each equal bit for bit (the array is smaller than the first call's
one-pass workspace, so that call also runs in segments, which gdn_prefill's contract makes
bitwise equal to one pass), and within the tolerances of the fp64 oracle.  A shape whose
single chunk does not fit in the array is rejected before anything is enqueued."""
import ctypes

import pytest
import torch

from linear_recurrent_attention_gated_amd import gdn
from linear_recurrent_attention_gated_amd.inputs import make_inputs
from tests.gpu_util import TOL_O, TOL_S, nrel, np32, oracle_prefill, say, to_dev

pytestmark = pytest.mark.gpu

# (B, T, Hk, Hv, dk, dv, chunk, dtype): the first needs ~81 MiB in one pass (> the 64 MiB
# array: two segments), the second a few MiB
CALLS = [(1, 4096, 16, 32, 128, 128, 64, torch.bfloat16),
         (2, 333, 2, 4, 64, 128, 32, torch.float32)]


def _run(d, chunk, noalloc):
    dd = to_dev(d)
    B, T, Hk, dk = dd["q"].shape
    Hv, dv = dd["v"].shape[2], dd["v"].shape[3]
    o = torch.empty((B, T, Hv, dv), dtype=dd["q"].dtype, device="cuda")
    s = torch.empty((B, Hv, dv, dk), dtype=torch.float32, device="cuda")
    st = dd["state"]
    if noalloc:
        gdn.gdn_prefill_noalloc(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], st, o, s, chunk)
    else:
        nb = gdn.gdn_prefill_workspace_bytes(B, T, Hk, Hv, dk, dv, chunk, dd["q"].dtype)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        gdn.gdn_prefill(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], st, o, s, chunk, ws)
    torch.cuda.synchronize()
    return o, s


def test_noalloc_prefill_equals_gdn_prefill_twice_in_a_row():
    full = gdn.gdn_prefill_workspace_bytes(*CALLS[0][:7], torch.bfloat16)
    assert full > gdn.NOALLOC_SCRATCH_BYTES
    results = []
    for i, (B, T, Hk, Hv, dk, dv, chunk, dt) in enumerate(CALLS):
        d = make_inputs(B, T, Hk, Hv, dk, dv, seed=60 + i, dtype=dt, state_std=0.1)
        say("noalloc call", i, (B, T, Hk, Hv, dk, dv, chunk, dt))
        o1, s1 = _run(d, chunk, noalloc=True)
        results.append((d, chunk, o1, s1))
    for i, (d, chunk, o1, s1) in enumerate(results):
        say("gdn_prefill reference", i)
        o2, s2 = _run(d, chunk, noalloc=False)
        assert torch.equal(o1, o2) and torch.equal(s1, s2), i
        o_ref, s_ref = oracle_prefill(d, d["state"], nthreads=16)
        eo, es = nrel(np32(o1), o_ref), nrel(s1.cpu().numpy(), s_ref)
        say("noalloc errors", i, eo, es)
        assert eo < TOL_O and es < TOL_S


def test_noalloc_rejects_a_chunk_larger_than_the_array():
    # one 64-token chunk at B = 64, 16/32 heads, d = 128 needs ~84 MB of blocks
    L = gdn.lib()
    B, T, Hk, Hv, dk, dv, C = 64, 64, 16, 32, 128, 128, 64
    per_call = gdn.gdn_prefill_workspace_bytes(B, T, Hk, Hv, dk, dv, C, torch.bfloat16)
    assert per_call > gdn.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, T, Hk, dk), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((B, T, Hv, dv), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((B, T, Hv), dtype=torch.float32, device="cuda")
    s = torch.zeros((B, Hv, dv, dk), dtype=torch.float32, device="cuda")
    o = torch.empty_like(v)
    rc = L.gdn_prefill_noalloc(q.data_ptr(), q.data_ptr(), v.data_ptr(), g.data_ptr(),
                               g.data_ptr(), None, o.data_ptr(), s.data_ptr(), B, T, Hk, Hv,
                               dk, dv, C, 0, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 6   # GDN_ERR_WORKSPACE
