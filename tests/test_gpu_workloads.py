"""GPU parity at the full workload sizes, in the launch configuration the benchmark
times, plus the properties the pages state or the method implies.

Full sizes, each in the bf16 build (bf16 q/k/v/o, fp32 gates and state) and in the
all-fp32 build, every value head against the oracle: the 4096-token prefill, the
32768-token continuation from a nonzero state, the 131072-token long-memory prefill
and its prefix sweep, and one decode token through 30 layers (looped and batched).

Properties: segmenting a prompt and carrying the state gives the same output
("Optimizing on-device inference for Apple Silicon", section "Bound temporary
memory with prompt chunking"); key heads shared 2:1 give the same bytes as the
duplicated heads (section "Pack query heads to reuse KV rows" makes the same
point for attention); chunk size does not change the result; a one-token prefill
equals a decode step; repeated runs are bitwise identical.
"""
import numpy as np
import pytest
import torch

from linear_recurrent_attention_gated_amd import gdn
from linear_recurrent_attention_gated_amd.inputs import (CONTINUATION_32K, LONG_128K, PREFILL_4K,
                                                         DECODE_LAYERS, decode_inputs,
                                                         make_inputs, workload_inputs)
from tests.gpu_util import TOL_O, TOL_S, nrel, np32, oracle_prefill, say, to_dev

pytestmark = pytest.mark.gpu

NTHREADS = 16


def gpu_prefill(d, chunk, state=None, dtype_ws=None):
    dd = to_dev(d)
    st = None if state is None else torch.as_tensor(np.asarray(state, np.float32)).cuda()
    o, s = gdn.prefill(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], st, chunk=chunk)
    torch.cuda.synchronize()
    return o, s


DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def per_head_errors(o_g, s_g, o_ref, s_ref, heads):
    """Normwise errors of every value head (each head is an independent recurrence, so each
    is held to the tolerance on its own); returns the worst pair."""
    worst_o = worst_s = 0.0
    for i, h in enumerate(heads):
        eo, es = nrel(o_g[0, :, h], o_ref[0, :, i]), nrel(s_g[0, h], s_ref[0, i])
        worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
        assert eo < TOL_O and es < TOL_S, (h, eo, es)
    return worst_o, worst_s


@pytest.fixture(scope="module", params=sorted(DTYPES))
def c2(request):
    """The 4096-token prefill workload and its oracle result, in either build."""
    dt = request.param
    d = workload_inputs(PREFILL_4K, DTYPES[dt])
    o_ref, s_ref = oracle_prefill(d, nthreads=NTHREADS)
    return dt, d, o_ref, s_ref


def test_prefill_4k_all_heads(c2):
    w = PREFILL_4K
    dt, d, o_ref, s_ref = c2
    say("prefill 4k", dt)
    o, s = gpu_prefill(d, w.chunk)
    eo, es = nrel(np32(o), o_ref), nrel(s.cpu().numpy(), s_ref)
    say("prefill 4k errors", dt, eo, es)
    assert eo < TOL_O and es < TOL_S


def test_continuation_32k_from_nonzero_state(c2):
    # every value head of the 32768-token continuation against the oracle, from the oracle's
    # final state of the 4096-token prefill (same build), then the GPU's own chained result
    w = CONTINUATION_32K
    dt, d0, _, s_c2 = c2
    start = s_c2.astype(np.float32)
    d = workload_inputs(w, DTYPES[dt])
    say("continuation 32k", dt)
    o, s = gpu_prefill(d, w.chunk, start)
    o_ref, s_ref = oracle_prefill(d, start.astype(np.float64), nthreads=NTHREADS)
    o_g, s_g = np32(o), s.cpu().numpy()
    heads = list(range(w.Hv))
    o_ref = o_ref.reshape(1, w.T, w.Hv, w.dv)
    eo, es = per_head_errors(o_g, s_g, o_ref, s_ref, heads)
    say("continuation 32k worst head errors", dt, eo, es)
    # chained on the GPU: its own 4096-token state carried into the continuation
    _, s_gpu_c2 = gpu_prefill(d0, PREFILL_4K.chunk)
    o2, s2 = gpu_prefill(d, w.chunk, s_gpu_c2.cpu().numpy())
    eo2, es2 = per_head_errors(np32(o2), s2.cpu().numpy(), o_ref, s_ref, heads)
    say("continuation 32k chained worst head errors", dt, eo2, es2)


@pytest.fixture(scope="module", params=sorted(DTYPES))
def c4(request):
    dt = request.param
    d = workload_inputs(LONG_128K, DTYPES[dt])
    say("long 128k: GPU run", dt)
    o, s = gpu_prefill(d, LONG_128K.chunk)
    return dt, d, np32(o), s.cpu().numpy()


def test_long_128k_all_heads(c4):
    # the fixed-size state carries 131072 tokens of long-memory gates (a near 1): the longest
    # accumulation of rounding in the fp32 state of either build, checked on every value head
    dt, d, o_g, s_g = c4
    w = LONG_128K
    say("long 128k oracle", dt)
    o_ref, s_ref = oracle_prefill(d, nthreads=NTHREADS)
    assert np.all(np.isfinite(o_g)) and np.all(np.isfinite(s_g))
    eo, es = per_head_errors(o_g, s_g, o_ref.reshape(1, w.T, w.Hv, w.dv), s_ref, list(range(w.Hv)))
    say("long 128k worst head errors", dt, eo, es)


def test_long_sweep_prefixes(c4):
    # the sweep T = 256, 512, ..., 65536 runs prefixes of the same draw; chunk-aligned prefixes
    # go through identical chunk computations, so their outputs equal the full run's bitwise
    dt, d, o_full, _ = c4
    for T in [256 << i for i in range(9)]:
        dp = {k: (None if v is None else v[:, :T].contiguous()) for k, v in d.items()}
        say("sweep prefix", dt, T)
        o, _ = gpu_prefill(dp, LONG_128K.chunk)
        assert np.array_equal(np32(o), o_full[:, :T]), T


@pytest.mark.parametrize("dt", sorted(DTYPES))
def test_decode_30_layers_looped_and_batched(dt):
    # one token through 30 independent layers at 16 key / 32 value heads, d = 128: 30 B = 1
    # launches and one B = 30 launch give the same bits, and every layer meets the tolerance
    dtype = DTYPES[dt]
    layers = [decode_inputs(l, dtype) for l in range(DECODE_LAYERS)]
    cat = {k: torch.cat([L[k] for L in layers]).cuda() for k in layers[0]}
    st_loop = cat["state"].clone()
    st_b = cat["state"].clone()
    o_loop = torch.empty((DECODE_LAYERS, 32, 128), dtype=dtype, device="cuda")
    o_b = torch.empty_like(o_loop)
    say("decode 30 layers", dt)
    for l in range(DECODE_LAYERS):
        sl = slice(l, l + 1)
        gdn.gdn_decode_step(cat["q"][sl], cat["k"][sl], cat["v"][sl], cat["g"][sl],
                            cat["beta"][sl], st_loop[sl], st_loop[sl], o_loop[sl])
    gdn.gdn_decode_step(cat["q"], cat["k"], cat["v"], cat["g"], cat["beta"], st_b, st_b, o_b)
    torch.cuda.synchronize()
    assert torch.equal(st_loop, st_b) and torch.equal(o_loop, o_b)
    f = lambda t: t.float().numpy()  # noqa: E731
    from oracle import gdn_oracle as orc
    o_ref, s_ref = orc.decode_step(f(cat["q"].cpu()), f(cat["k"].cpu()), f(cat["v"].cpu()),
                                   f(cat["g"].cpu()), f(cat["beta"].cpu()),
                                   cat["state"].cpu().numpy().astype(np.float64))
    worst_o = worst_s = 0.0
    for l in range(DECODE_LAYERS):
        eo, es = nrel(np32(o_loop[l]), o_ref[l]), nrel(st_loop[l].cpu().numpy(), s_ref[l])
        worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
        assert eo < TOL_O and es < 1e-6, (l, eo, es)
    say("decode 30 layers worst layer errors", dt, worst_o, worst_s)


def test_split_invariance_state_carry():
    d = make_inputs(1, 1000, 2, 4, 128, 128, seed=21, state_std=0.2)
    o_full, s_full = gpu_prefill(d, 64, d["state"])
    for T1 in (1, 64, 333):
        a = {k: (v if k == "state" else v[:, :T1].contiguous()) for k, v in d.items()}
        b = {k: (v if k == "state" else v[:, T1:].contiguous()) for k, v in d.items()}
        say("split", T1)
        oa, sa = gpu_prefill(a, 64, d["state"])
        ob, sb = gpu_prefill(b, 64, sa.cpu().numpy())
        o_cat = torch.cat([oa, ob], dim=1)
        assert nrel(np32(o_cat), np32(o_full)) < 1e-2 and nrel(sb.cpu().numpy(), s_full.cpu().numpy()) < 5e-3
        if T1 == 64:   # a chunk-aligned split runs the very same chunk computations
            assert torch.equal(o_cat, o_full) and torch.equal(sb, s_full)


def test_chunk_size_invariance():
    d = make_inputs(1, 300, 2, 4, 64, 128, seed=22, state_std=0.2)
    ref_o, ref_s = oracle_prefill(d, d["state"])
    outs = {}
    for C in (16, 32, 64):
        say("chunk", C)
        o, s = gpu_prefill(d, C, d["state"])
        outs[C] = (np32(o), s.cpu().numpy())
        assert nrel(outs[C][0], ref_o) < TOL_O and nrel(outs[C][1], ref_s) < TOL_S
    assert nrel(outs[16][0], outs[64][0]) < 2e-2


def test_single_token_prefill_equals_decode():
    d = make_inputs(2, 1, 16, 32, 128, 128, seed=23, state_std=0.1)
    o_p, s_p = gpu_prefill(d, 64, d["state"])
    dd = to_dev(d)
    st = dd["state"].clone()
    say("T=1 vs decode")
    o_d = gdn.decode_step(dd["q"][:, 0].contiguous(), dd["k"][:, 0].contiguous(),
                          dd["v"][:, 0].contiguous(), dd["g"][:, 0].contiguous(),
                          dd["beta"][:, 0].contiguous(), st)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(d, d["state"])
    # both paths meet the tolerances against the oracle; the decode step (fp32 throughout)
    # is far tighter on the state than the blockwise form (bf16 matrix-core operands)
    assert nrel(np32(o_p), o_ref) < TOL_O and nrel(s_p.cpu().numpy(), s_ref) < TOL_S
    assert nrel(np32(o_d), o_ref[:, 0]) < TOL_O and nrel(st.cpu().numpy(), s_ref) < 1e-6
    assert nrel(np32(o_p[:, 0]), np32(o_d)) < TOL_O


def test_many_workgroups_large_batch():
    # 16 prompts of 96 tokens (a ragged second chunk) at 16/32 heads: 4,096 scan workgroups and
    # 1,024 intra items, so the XCD-aware placement and the persistent intra grid run far past
    # one workgroup per CU; sampled (batch, value head) pairs against the oracle
    B, T = 16, 96
    h = make_inputs(B, T, 16, 32, 128, 128, seed=29, state_std=0.2)
    say("many workgroups", B, T)
    o, s = gpu_prefill(h, 64, state=h["state"])
    pairs = [(0, 0), (3, 7), (7, 31), (8, 16), (12, 5), (15, 30)]
    o_ref, s_ref = oracle_prefill(h, h["state"], pairs=pairs, nthreads=NTHREADS)
    og, sg = np32(o), s.cpu().numpy()
    for i, (b, hv) in enumerate(pairs):
        eo, es = nrel(og[b, :, hv], o_ref[i]), nrel(sg[b, hv], s_ref[i])
        assert eo < TOL_O and es < TOL_S, (b, hv, eo, es)


def test_shared_key_heads_equal_duplicated_heads_bitwise():
    d = make_inputs(1, 200, 16, 32, 128, 128, seed=24)
    dup = dict(d)
    dup["q"] = d["q"].repeat_interleave(2, dim=2).contiguous()
    dup["k"] = d["k"].repeat_interleave(2, dim=2).contiguous()
    say("shared vs duplicated heads")
    o1, s1 = gpu_prefill(d, 64)
    o2, s2 = gpu_prefill(dup, 64)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_bitwise_deterministic():
    d = make_inputs(1, 777, 2, 4, 128, 128, seed=25, state_std=0.1)
    say("determinism")
    o1, s1 = gpu_prefill(d, 64, d["state"])
    o2, s2 = gpu_prefill(d, 64, d["state"])
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def _prefill_with_workspace(d, chunk, nbytes, state=None):
    dd = to_dev(d)
    B, T, Hk, dk = dd["q"].shape
    Hv, dv = dd["v"].shape[2], dd["v"].shape[3]
    o = torch.empty((B, T, Hv, dv), dtype=dd["q"].dtype, device="cuda")
    s_out = torch.empty((B, Hv, dv, dk), dtype=torch.float32, device="cuda")
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    st = None if state is None else torch.as_tensor(np.asarray(state, np.float32)).cuda()
    gdn.gdn_prefill(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], st, o, s_out, chunk, ws)
    torch.cuda.synchronize()
    return o, s_out


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("chunk,seg_chunks", [(64, 1), (64, 3), (32, 5), (16, 7)])
def test_segmented_prefill_equals_one_pass(dt, chunk, seg_chunks):
    # "Bound temporary memory with prompt chunking": a workspace that holds only seg_chunks
    # chunks makes gdn_prefill run the prompt in segments, carrying the state between them;
    # every chunk computation is the same as in one pass, so the result is identical
    d = make_inputs(2, 1000, 2, 4, 128, 128, seed=26, state_std=0.1, dtype=dt)
    full = gdn.gdn_prefill_workspace_bytes(2, 1000, 2, 4, 128, 128, chunk, dt)
    small = gdn.gdn_prefill_workspace_bytes(2, seg_chunks * chunk, 2, 4, 128, 128, chunk, dt)
    assert small < full
    say("segmented", dt, chunk, seg_chunks)
    o1, s1 = _prefill_with_workspace(d, chunk, full, d["state"])
    o2, s2 = _prefill_with_workspace(d, chunk, small, d["state"])
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    o_ref, s_ref = oracle_prefill(d, d["state"])
    assert nrel(np32(o2), o_ref) < TOL_O and nrel(s2.cpu().numpy(), s_ref) < TOL_S


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_prepare_then_scan_equals_one_call(dt):
    # gdn_prefill is gdn_prefill_prepare followed by gdn_prefill_scan on one workspace: the two
    # stages called separately (the scan also reads v itself) give the same bits, also when
    # another call's stages ran on a second workspace in between
    d = make_inputs(1, 300, 2, 4, 128, 128, seed=41, state_std=0.1, dtype=dt)
    e = make_inputs(1, 300, 2, 4, 128, 128, seed=42, state_std=0.1, dtype=dt)
    dd, de = to_dev(d), to_dev(e)
    nbytes = gdn.gdn_prefill_workspace_bytes(1, 300, 2, 4, 128, 128, 64, dt)
    ws1 = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    st = torch.as_tensor(np.asarray(d["state"], np.float32)).cuda()
    ste = torch.as_tensor(np.asarray(e["state"], np.float32)).cuda()
    o1 = torch.empty_like(dd["v"])
    s1 = torch.empty((1, 4, 128, 128), dtype=torch.float32, device="cuda")
    o2, s2 = torch.empty_like(o1), torch.empty_like(s1)
    oe, se = torch.empty_like(o1), torch.empty_like(s1)
    say("prepare+scan", dt)
    args = (dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], st)
    gdn.gdn_prefill(*args, o1, s1, 64, ws1)
    gdn.gdn_prefill_prepare(*args, o2, s2, 64, ws1)
    gdn.gdn_prefill_prepare(de["q"], de["k"], de["v"], de["g"], de["beta"], ste, oe, se, 64, ws2)
    gdn.gdn_prefill_scan(de["q"], de["k"], de["v"], de["g"], de["beta"], ste, oe, se, 64, ws2)
    gdn.gdn_prefill_scan(*args, o2, s2, 64, ws1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    o_ref, s_ref = oracle_prefill(e, e["state"])
    assert nrel(np32(oe), o_ref) < TOL_O and nrel(se.cpu().numpy(), s_ref) < TOL_S


@pytest.mark.parametrize("dt,T,B", [(torch.bfloat16, 8292, 1), (torch.float32, 12100, 1),
                                    (torch.bfloat16, 4100, 2)])
def test_cache_sized_passes_equal_one_pass(dt, T, B):
    # at 16/32 heads and d = 128 these prompts exceed one pass's last-level-cache budget (the
    # batch of two at 4K too: the budget covers the whole batch), so gdn_prefill runs them in
    # equal passes even with the one-pass workspace; the two stages called separately always
    # make one pass: the results must be bitwise equal
    h = make_inputs(B, T, 16, 32, 128, 128, seed=27 + B, state_std=0.1, dtype=dt)
    d = to_dev(h)
    nbytes = gdn.gdn_prefill_workspace_bytes(B, T, 16, 32, 128, 128, 64, dt)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o1, o2 = torch.empty_like(d["v"]), torch.empty_like(d["v"])
    s1 = torch.empty((B, 32, 128, 128), dtype=torch.float32, device="cuda")
    s2 = torch.empty_like(s1)
    say("cache-sized passes", dt, T, B)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"])
    gdn.gdn_prefill(*args, o1, s1, 64, ws)
    gdn.gdn_prefill_prepare(*args, o2, s2, 64, ws)
    gdn.gdn_prefill_scan(*args, o2, s2, 64, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    if B > 1:   # and the batch against the oracle, every (batch, value head)
        o_ref, s_ref = oracle_prefill(h, h["state"], nthreads=NTHREADS)
        og, sg = np32(o1), s1.cpu().numpy()
        for b in range(B):
            for hv in range(32):
                eo, es = nrel(og[b, :, hv], o_ref[b, :, hv]), nrel(sg[b, hv], s_ref[b, hv])
                assert eo < TOL_O and es < TOL_S, (b, hv, eo, es)


def test_long_128k_bounded_workspace(c4):
    # the 131072-token prompt with a 256 MiB workspace (the one-pass workspace is 2.5-5 GiB)
    dt, d, o_full, s_full = c4
    w = LONG_128K
    full = gdn.gdn_prefill_workspace_bytes(w.B, w.T, w.Hk, w.Hv, w.dk, w.dv, w.chunk, DTYPES[dt])
    assert full > 8 * (256 << 20)
    say("long 128k, bounded workspace", dt)
    o, s = _prefill_with_workspace(d, w.chunk, 256 << 20)
    assert np.array_equal(np32(o), o_full) and np.array_equal(s.cpu().numpy(), s_full)
