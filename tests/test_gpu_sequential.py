"""GPU parity of the token-sequential prefill (gdn_prefill_ex with GDN_PATH_SEQUENTIAL)
against the fp64 oracle, and of the automatic choice between the two forms.

The sequential form runs in fp32 throughout (bf16 inputs widened exactly), so its
errors are far below the bf16-MFMA blockwise form's; both are held to the same
tolerances, and the all-fp32 cases to 1e-4."""
import numpy as np
import pytest
import torch

from linear_recurrent_attention_gated_amd import gdn
from linear_recurrent_attention_gated_amd.inputs import make_inputs
from tests.gpu_util import TOL_O, TOL_S, nrel, np32, oracle_prefill, say, to_dev

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f32": torch.float32}

CASES = [
    # B, T, Hk, Hv, dk, dv, with_state
    (1, 1, 1, 1, 32, 32, False),
    (1, 7, 1, 2, 32, 64, True),
    (2, 17, 2, 4, 64, 32, True),
    (1, 63, 1, 1, 128, 128, False),
    (1, 100, 2, 4, 128, 64, True),
    (2, 129, 1, 2, 64, 128, True),
    (1, 300, 2, 4, 32, 128, True),
    (1, 520, 1, 2, 128, 128, True),
    (3, 33, 1, 4, 64, 64, True),
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("qk_norm", [False, True], ids=["plain", "qknorm"])
@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}T{c[1]}h{c[2]}-{c[3]}d{c[4]}x{c[5]}"
                                             + ("s" if c[6] else "") for c in CASES])
def test_sequential_matches_oracle(case, qk_norm, dt):
    B, T, Hk, Hv, dk, dv, with_state = case
    d = make_inputs(B, T, Hk, Hv, dk, dv, seed=3000 + T, dtype=DT[dt],
                    state_std=0.3 if with_state else None, unit_qk=not qk_norm)
    dd = to_dev(d)
    say("sequential", dt, qk_norm, case)
    o, s = gdn.prefill(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["state"], chunk=64,
                       qk_norm=qk_norm, path="sequential")
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(d, d["state"], qk_norm=qk_norm)
    eo, es = nrel(np32(o), o_ref), nrel(s.cpu().numpy(), s_ref)
    say("sequential errors", dt, qk_norm, case, eo, es)
    assert eo < TOL_O and es < TOL_S
    # fp32 arithmetic on exact inputs: only the output's own rounding is visible in bf16
    assert es < 1e-4 and eo < (1e-4 if dt == "f32" else 8e-3)


def test_sequential_in_place_state_and_no_workspace():
    d = make_inputs(1, 90, 2, 4, 64, 64, seed=31, state_std=0.5)
    dd = to_dev(d)
    ref_o, ref_s = oracle_prefill(d, d["state"])
    st = dd["state"].clone()
    o = torch.empty_like(dd["v"])
    say("sequential in place, no workspace")
    gdn.gdn_prefill_ex(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], st, o, st, 64, None,
                       gdn.GDN_PATH_SEQUENTIAL)
    torch.cuda.synchronize()
    assert nrel(np32(o), ref_o) < TOL_O and nrel(st.cpu().numpy(), ref_s) < TOL_S


def test_sequential_strong_decay_and_reset():
    d = make_inputs(1, 200, 1, 2, 128, 128, seed=32, g_mean=3.0, state_std=1.0)
    d["g"][0, 120, :] = -30.0
    dd = to_dev(d)
    say("sequential strong decay")
    o, s = gdn.prefill(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["state"],
                       path="sequential")
    torch.cuda.synchronize()
    o, s = np32(o), s.cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    o_ref, s_ref = oracle_prefill(d, d["state"])
    assert nrel(o, o_ref) < TOL_O and nrel(s, s_ref) < TOL_S


@pytest.mark.parametrize("qk_norm", [False, True], ids=["plain", "qknorm"])
def test_auto_picks_by_length(qk_norm):
    # at or below the crossover the automatic choice is the sequential form, above it the
    # blockwise form: bitwise equal to the chosen form's own output
    Hk, Hv, dk, dv = 2, 4, 128, 128
    lim = gdn.gdn_prefill_sequential_max_tokens(1, Hk, Hv, dk, dv, torch.bfloat16)
    assert lim >= 1
    for T, expect in ((lim, "sequential"), (lim + 1, "blockwise")):
        d = to_dev(make_inputs(1, T, Hk, Hv, dk, dv, seed=33, state_std=0.2,
                               unit_qk=not qk_norm))
        say("auto", T, expect, qk_norm)
        oa, sa = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], chunk=64,
                             qk_norm=qk_norm, path="auto")
        oe, se = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], chunk=64,
                             qk_norm=qk_norm, path=expect)
        torch.cuda.synchronize()
        assert torch.equal(oa, oe) and torch.equal(sa, se), (T, expect)


@pytest.mark.parametrize("qk_norm", [False, True], ids=["plain", "qknorm"])
def test_auto_one_token_is_the_decode_step(qk_norm):
    # one token from a given state: the automatic choice is the decode step, bitwise equal to
    # gdn_decode_step on the same (T = 1) tensors, and within the oracle's tolerances; without
    # a start state it stays the sequential form
    Hk, Hv, dk, dv = 2, 4, 128, 64
    h = make_inputs(2, 1, Hk, Hv, dk, dv, seed=34, state_std=0.2, unit_qk=not qk_norm)
    d = to_dev(h)
    say("auto one token", qk_norm)
    oa, sa = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], chunk=64,
                         qk_norm=qk_norm, path="auto")
    st = d["state"].clone()
    od = gdn.decode_step(d["q"][:, 0].contiguous(), d["k"][:, 0].contiguous(),
                         d["v"][:, 0].contiguous(), d["g"][:, 0].contiguous(),
                         d["beta"][:, 0].contiguous(), st, qk_norm=qk_norm)
    o0, s0 = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], None, chunk=64,
                         qk_norm=qk_norm, path="auto")
    o0s, s0s = gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], None, chunk=64,
                           qk_norm=qk_norm, path="sequential")
    torch.cuda.synchronize()
    assert torch.equal(oa[:, 0], od) and torch.equal(sa, st)
    assert torch.equal(o0, o0s) and torch.equal(s0, s0s)
    o_ref, s_ref = oracle_prefill(h, h["state"], qk_norm=qk_norm)
    assert nrel(np32(oa), o_ref) < TOL_O and nrel(sa.cpu().numpy(), s_ref) < TOL_S
