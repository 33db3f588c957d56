"""GPU parity of the fused query/key L2 normalisation (gdn_prefill_qknorm,
gdn_decode_step_qknorm) against the fp64 oracle's qk_norm scan, on raw
(unnormalised) q and k whose per-token lengths vary by a log-normal factor.

Covers both element types, every chunk size, ragged tails, a starting state, shared
key heads, zero query/key rows (the eps keeps them finite), the bounded-workspace
segmentation, and the decode step."""
import numpy as np
import pytest
import torch

from linear_recurrent_attention_gated_amd import gdn
from linear_recurrent_attention_gated_amd.inputs import make_inputs
from tests.gpu_util import TOL_O, TOL_S, nrel, np32, oracle_prefill, say, to_dev

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f32": torch.float32}

CASES = [
    # B, T, Hk, Hv, dk, dv, chunk, with_state
    (1, 1, 1, 1, 32, 32, 16, False),
    (2, 47, 2, 4, 64, 32, 16, True),
    (1, 95, 1, 2, 128, 64, 32, True),
    (1, 200, 2, 4, 128, 128, 64, True),
    (1, 130, 1, 1, 32, 128, 64, False),
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}T{c[1]}h{c[2]}-{c[3]}d{c[4]}x{c[5]}c{c[6]}"
                                             + ("s" if c[7] else "") for c in CASES])
def test_prefill_qknorm_matches_oracle(case, dt):
    B, T, Hk, Hv, dk, dv, chunk, with_state = case
    d = make_inputs(B, T, Hk, Hv, dk, dv, seed=2000 + T, dtype=DT[dt],
                    state_std=0.3 if with_state else None, unit_qk=False)
    dd = to_dev(d)
    say("prefill qknorm", dt, case)
    o, s = gdn.prefill(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["state"], chunk=chunk,
                       qk_norm=True)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(d, d["state"], qk_norm=True)
    eo, es = nrel(np32(o), o_ref), nrel(s.cpu().numpy(), s_ref)
    say("prefill qknorm errors", dt, case, eo, es)
    assert eo < TOL_O and es < TOL_S
    if dt == "f32":
        assert eo < 1e-4 and es < 1e-4


def test_prefill_qknorm_zero_rows_stay_finite():
    # zero keys leave only the decay, zero queries read zeros; rows inside a chunk and at its
    # boundaries
    d = make_inputs(1, 100, 2, 4, 64, 64, seed=21, state_std=0.5, unit_qk=False)
    for t in (0, 31, 32, 63, 77, 99):
        d["k"][0, t, t % 2] = 0
        d["q"][0, t, (t + 1) % 2] = 0
    dd = to_dev(d)
    say("prefill qknorm zero rows")
    o, s = gdn.prefill(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["state"], chunk=32,
                       qk_norm=True)
    torch.cuda.synchronize()
    o, s = np32(o), s.cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    o_ref, s_ref = oracle_prefill(d, d["state"], qk_norm=True)
    assert nrel(o, o_ref) < TOL_O and nrel(s, s_ref) < TOL_S


def test_prefill_qknorm_segmented_equals_one_pass():
    # per-token normalisation does not depend on where a segment starts: bitwise equal
    B, T, Hk, Hv, dk, dv, chunk = 1, 300, 2, 4, 64, 64, 32
    d = to_dev(make_inputs(B, T, Hk, Hv, dk, dv, seed=22, state_std=0.2, unit_qk=False))
    full = gdn.gdn_prefill_workspace_bytes(B, T, Hk, Hv, dk, dv, chunk, torch.bfloat16)
    small = gdn.gdn_prefill_workspace_bytes(B, 3 * chunk, Hk, Hv, dk, dv, chunk, torch.bfloat16)
    outs = []
    for nb in (full, small):
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        o = torch.empty_like(d["v"])
        s = torch.empty_like(d["state"])
        say("prefill qknorm workspace", nb)
        gdn.gdn_prefill_qknorm(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], o, s, chunk,
                               ws)
        torch.cuda.synchronize()
        outs.append((o.cpu(), s.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_prefill_qknorm_on_unit_inputs_matches_plain_prefill():
    # inputs already of unit length: normalising again changes them by O(eps) only
    d = to_dev(make_inputs(1, 160, 2, 4, 128, 128, seed=23, dtype=torch.float32, state_std=0.2))
    say("prefill qknorm vs plain on unit inputs")
    o1, s1 = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], chunk=64)
    o2, s2 = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], chunk=64,
                         qk_norm=True)
    torch.cuda.synchronize()
    assert nrel(np32(o2), np32(o1)) < 1e-5 and nrel(s2.cpu().numpy(), s1.cpu().numpy()) < 1e-5


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("dims", [(128, 128), (64, 32), (32, 128)])
def test_decode_qknorm_matches_oracle(dims, dt):
    dk, dv = dims
    B, Hk, Hv = 3, 2, 4
    d = make_inputs(B, 1, Hk, Hv, dk, dv, seed=30 + dk, dtype=DT[dt], state_std=0.1,
                    unit_qk=False)
    d["k"][1, 0, 1] = 0          # a zero key: decay only
    dd = to_dev(d)
    st = dd["state"].clone()
    say("decode qknorm", dt, dims)
    o = gdn.decode_step(dd["q"][:, 0].contiguous(), dd["k"][:, 0].contiguous(),
                        dd["v"][:, 0].contiguous(), dd["g"][:, 0].contiguous(),
                        dd["beta"][:, 0].contiguous(), st, qk_norm=True)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(d, d["state"], qk_norm=True)
    eo, es = nrel(np32(o), o_ref[:, 0]), nrel(st.cpu().numpy(), s_ref)
    say("decode qknorm errors", dt, dims, eo, es)
    assert eo < TOL_O and es < TOL_S
    assert es < 1e-6 and eo < (1e-5 if dt == "f32" else 8e-3)
