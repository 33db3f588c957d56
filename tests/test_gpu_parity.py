"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by
element, on seeded inputs.

Sizes span several chunks and ragged tails; head dimensions and head groupings
cover the compiled set; both element types (bf16 with an fp32 state, and all
fp32) are checked against the normwise tolerances (2e-2 on o, 1e-2 on the state).
"""
import numpy as np
import pytest
import torch

from linear_recurrent_attention_gated_amd import gdn
from linear_recurrent_attention_gated_amd.inputs import make_inputs, TINY
from tests.gpu_util import TOL_O, TOL_S, nrel, np32, oracle_prefill, say, to_dev

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def run_prefill(d, chunk, state=None):
    dd = to_dev(d)
    st = None if state is None else torch.as_tensor(state, dtype=torch.float32).cuda().contiguous()
    o, s = gdn.prefill(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], st, chunk=chunk)
    torch.cuda.synchronize()
    return np32(o), s.cpu().numpy()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_tiny_workload(dt):
    w = TINY
    d = make_inputs(w.B, w.T, w.Hk, w.Hv, w.dk, w.dv, w.seed, DT[dt])
    say("tiny", dt, w)
    o, s = run_prefill(d, w.chunk)
    o_ref, s_ref = oracle_prefill(d)
    eo, es = nrel(o, o_ref), nrel(s, s_ref)
    say("tiny errors", dt, eo, es)
    assert eo < TOL_O and es < TOL_S
    if dt == "f32":      # fp32 operands on fp32 matrix cores: far inside the tolerance
        assert eo < 1e-4 and es < 1e-4


CASES = [
    # B, T, Hk, Hv, dk, dv, chunk, with_state
    (1, 1, 1, 1, 32, 32, 16, False),
    (1, 15, 1, 2, 32, 64, 16, True),
    (2, 17, 2, 4, 64, 32, 16, True),
    (1, 63, 1, 1, 128, 128, 32, False),
    (1, 65, 2, 2, 64, 64, 64, True),
    (2, 100, 1, 2, 128, 64, 32, True),
    (1, 130, 2, 4, 32, 128, 64, True),
    (1, 257, 1, 2, 128, 128, 64, True),
    (1, 96, 3, 6, 64, 128, 16, True),
    (1, 200, 1, 1, 128, 32, 64, False),
    # four and eight value heads per key head, several batches
    (1, 150, 1, 4, 64, 64, 64, True),
    (2, 77, 2, 8, 128, 64, 32, True),
    (8, 40, 1, 4, 32, 32, 16, True),
    (1, 80, 1, 2, 128, 128, 16, True),
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}T{c[1]}h{c[2]}-{c[3]}d{c[4]}x{c[5]}c{c[6]}"
                                             + ("s" if c[7] else "") for c in CASES])
def test_prefill_matches_oracle(case, dt):
    B, T, Hk, Hv, dk, dv, chunk, with_state = case
    d = make_inputs(B, T, Hk, Hv, dk, dv, seed=1000 + T, dtype=DT[dt],
                    state_std=0.3 if with_state else None)
    say("prefill", dt, case)
    o, s = run_prefill(d, chunk, d["state"])
    o_ref, s_ref = oracle_prefill(d, d["state"])
    eo, es = nrel(o, o_ref), nrel(s, s_ref)
    say("prefill errors", dt, case, eo, es)
    assert eo < TOL_O and es < TOL_S
    if dt == "f32":
        assert eo < 1e-4 and es < 1e-4


def test_prefill_zero_length_copies_state():
    d = make_inputs(1, 1, 2, 4, 64, 32, seed=3, state_std=1.0)
    dd = to_dev(d)
    empty = lambda t: t[:, :0].contiguous()  # noqa: E731
    st = dd["state"].clone()
    out = torch.full_like(st, 7.0)
    o = torch.empty((1, 0, 4, 32), dtype=torch.bfloat16, device="cuda")
    say("prefill T=0")
    gdn.gdn_prefill(empty(dd["q"]), empty(dd["k"]), empty(dd["v"]), empty(dd["g"]),
                    empty(dd["beta"]), st, o, out, 16, None)
    torch.cuda.synchronize()
    assert torch.equal(out, st)
    gdn.gdn_prefill(empty(dd["q"]), empty(dd["k"]), empty(dd["v"]), empty(dd["g"]),
                    empty(dd["beta"]), None, o, out, 16, None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


def test_prefill_in_place_state():
    d = make_inputs(1, 80, 2, 4, 64, 64, seed=4, state_std=0.5)
    dd = to_dev(d)
    ref_o, ref_s = oracle_prefill(d, d["state"])
    st = dd["state"].clone()
    o = torch.empty_like(dd["v"])
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(1, 80, 2, 4, 64, 64, 32, 0),
                     dtype=torch.uint8, device="cuda")
    say("prefill in place")
    gdn.gdn_prefill(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], st, o, st, 32, ws)
    torch.cuda.synchronize()
    assert nrel(np32(o), ref_o) < TOL_O and nrel(st.cpu().numpy(), ref_s) < TOL_S


def test_strong_decay_and_reset_gates():
    # gates far below -88 per chunk (exp underflows in fp32) and an isolated reset g = -30
    d = make_inputs(1, 128, 1, 2, 64, 64, seed=5, g_mean=3.0, state_std=1.0)
    d["g"][0, 70, :] = -30.0
    say("strong decay")
    o, s = run_prefill(d, 64, d["state"])
    o_ref, s_ref = oracle_prefill(d, d["state"])
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    assert nrel(o, o_ref) < TOL_O and nrel(s, s_ref) < TOL_S


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("dims", [(128, 128), (64, 32), (32, 128), (64, 64, 1, 8)])
def test_decode_matches_oracle(dims, dt):
    dk, dv = dims[:2]
    B, Hk, Hv = (3, 2, 4) if len(dims) == 2 else (2,) + tuple(dims[2:])
    d = make_inputs(B, 1, Hk, Hv, dk, dv, seed=7 + dk, dtype=DT[dt], state_std=0.1)
    say("decode", dt, dims)
    dd = to_dev(d)
    st = dd["state"].clone()
    o = gdn.decode_step(dd["q"][:, 0].contiguous(), dd["k"][:, 0].contiguous(),
                        dd["v"][:, 0].contiguous(), dd["g"][:, 0].contiguous(),
                        dd["beta"][:, 0].contiguous(), st)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(d, d["state"])
    eo, es = nrel(np32(o), o_ref[:, 0]), nrel(st.cpu().numpy(), s_ref)
    say("decode errors", dt, dims, eo, es)
    assert eo < TOL_O and es < TOL_S
    # fp32 VALU on exact inputs: rounding only (plus the bf16 rounding of o itself)
    assert es < 1e-6 and eo < (1e-5 if dt == "f32" else 8e-3)


def test_decode_out_of_place_leaves_input():
    d = make_inputs(1, 1, 16, 32, 128, 128, seed=9, state_std=0.1)
    dd = to_dev(d)
    sin = dd["state"].clone()
    sout = torch.empty_like(sin)
    o = torch.empty((1, 32, 128), dtype=torch.bfloat16, device="cuda")
    say("decode out of place")
    gdn.gdn_decode_step(dd["q"][:, 0].contiguous(), dd["k"][:, 0].contiguous(),
                        dd["v"][:, 0].contiguous(), dd["g"][:, 0].contiguous(),
                        dd["beta"][:, 0].contiguous(), sin, sout, o)
    torch.cuda.synchronize()
    assert torch.equal(sin, dd["state"])
    o_ref, s_ref = oracle_prefill(d, d["state"])
    assert nrel(sout.cpu().numpy(), s_ref) < 1e-6 and nrel(np32(o), o_ref[:, 0]) < TOL_O
