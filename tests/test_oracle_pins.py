"""Pins for the CPU oracle: each test ties it to something other than itself.

The pages ("Optimizing on-device inference for Apple Silicon") print no numeric
example of the recurrence, so the pins are: exact rational arithmetic, closed
forms of special cases (write-then-read with orthonormal keys, pure decay, pure
readout, the single-token update, gated linear attention for mutually
orthogonal keys), the unrolled product form of the state, invariants the pages
state (segmenting a prompt does not change the output -- section "Bound
temporary memory with prompt chunking"; packing heads that share a key gives
identical bytes -- section "Pack query heads to reuse KV rows"), a norm bound,
and the blockwise form against the token scan (section "Qwen creates three
distinct workload shapes": the same computation evaluated two ways).

Shapes use dk != dv and Hv = 2 Hk so a transposed state or a wrong head
mapping cannot pass.
"""
import json
import os

import numpy as np
import pytest

from oracle import gdn_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "exact_tiny.json")


def rand_inputs(seed, B=1, T=12, Hk=1, Hv=2, dk=6, dv=4, unit=True, g_scale=1.0,
                beta_range=(0.05, 0.95), state=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, Hk, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, Hk, dk)).astype(np.float32)
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, Hv, dv)).astype(np.float32)
    g = (-g_scale * rng.random((B, T, Hv))).astype(np.float32)
    beta = rng.uniform(*beta_range, size=(B, T, Hv)).astype(np.float32)
    S0 = rng.standard_normal((B, Hv, dv, dk)) if state else None
    return q, k, v, g, beta, S0


def rel(x, ref):
    return np.max(np.abs(np.asarray(x) - ref)) / max(np.max(np.abs(ref)), 1e-300)


# --- exact rational golden values -----------------------------------------------------------

def test_exact_golden_fixture():
    doc = json.load(open(GOLDEN))
    for c in doc["cases"]:
        T, dk, dv = c["T"], c["dk"], c["dv"]
        q = np.array(c["q"], np.float32).reshape(1, T, 1, dk)
        k = np.array(c["k"], np.float32).reshape(1, T, 1, dk)
        v = np.array(c["v"], np.float32).reshape(1, T, 1, dv)
        g = np.array(c["g"], np.float32).reshape(1, T, 1)
        beta = np.array(c["beta"], np.float32).reshape(1, T, 1)
        S0 = None if c["state_in"] is None else np.array(c["state_in"]).reshape(1, 1, dv, dk)
        o_ref = np.array(c["o"]).reshape(1, T, 1, dv)
        s_ref = np.array(c["state_out"]).reshape(1, 1, dv, dk)
        for fn in (orc.seq, orc.seq_literal):
            o, s = fn(q, k, v, g, beta, S0)
            assert rel(o, o_ref) < 1e-13, fn.__name__
            assert rel(s, s_ref) < 1e-13, fn.__name__
        for C in (1, 2, 4, 16):
            o, s = orc.chunked(q, k, v, g, beta, S0, chunk=C)
            assert rel(o, o_ref) < 1e-12 and rel(s, s_ref) < 1e-12, C


# --- P1: rank-1 scan (C) against the literal matrix formula ---------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_p1_rank1_matches_literal(seed):
    q, k, v, g, beta, S0 = rand_inputs(seed, B=2, T=9, state=True, unit=(seed != 2))
    o1, s1 = orc.seq(q, k, v, g, beta, S0)
    o2, s2 = orc.seq_literal(q, k, v, g, beta, S0)
    assert rel(o1, o2) < 1e-13 and rel(s1, s2) < 1e-13


# --- P2: write-then-read ---------------------------------------------------------------------

def test_p2_write_then_read_orthonormal_keys():
    rng = np.random.default_rng(5)
    dk, dv, T = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:, :T].T.astype(np.float32)               # T orthonormal rows (rounded to fp32)
    k = keys.reshape(1, T, 1, dk)
    q = k.copy()
    v = rng.standard_normal((1, T, 1, dv)).astype(np.float32)
    g = np.zeros((1, T, 1), np.float32)                 # a = 1
    beta = np.ones((1, T, 1), np.float32)               # beta = 1
    o, S = orc.seq(q, k, v, g, beta)
    # every stored association reads back: S_T k_s = v_s
    kd = keys.astype(np.float64)
    for s in range(T):
        np.testing.assert_allclose(S[0, 0] @ kd[s], v[0, s, 0], atol=1e-6)
    # with beta = 1 and a unit key, reading the just-written key returns its value
    np.testing.assert_allclose(o[0, :, 0], v[0, :, 0], atol=1e-6)


def test_p2b_read_back_any_gate_any_state():
    # beta = 1, |k_t| = 1 (exactly, in fp64 arithmetic on the stored fp32 key), q_t = k_t
    # => o_t = S_t k_t = v_t whatever a_t and S_{t-1} are.
    q, k, v, g, beta, S0 = rand_inputs(7, T=10, state=True, g_scale=3.0)
    kd = k.astype(np.float64)
    kd /= np.linalg.norm(kd, axis=-1, keepdims=True)
    beta[:] = 1.0
    o, _ = orc.seq_literal(kd, kd, v, g, beta, S0)     # fp64 unit keys
    np.testing.assert_allclose(o[:, :, :, :], np.repeat(v[:, :, :, :], 1, 2).astype(np.float64),
                               atol=1e-12)
    o2, _ = orc.seq(k, k, v, g, beta, S0)               # fp32-stored keys: |k| = 1 +- 1e-7
    np.testing.assert_allclose(o2, v.astype(np.float64), atol=1e-5)


# --- P3/P4: pure decay and pure readout ------------------------------------------------------

def test_p3_beta_zero_pure_decay():
    q, k, v, g, beta, S0 = rand_inputs(3, B=2, T=11, state=True, g_scale=0.7)
    beta[:] = 0.0
    o, S = orc.seq(q, k, v, g, beta, S0)
    cum = np.cumsum(g.astype(np.float64), axis=1)         # log prod_{s<=t} a_s
    Hv, grp = v.shape[2], v.shape[2] // q.shape[2]
    for b in range(2):
        for h in range(Hv):
            np.testing.assert_allclose(S[b, h], np.exp(cum[b, -1, h]) * S0[b, h], rtol=1e-13)
            for t in range(11):
                ref = np.exp(cum[b, t, h]) * (S0[b, h] @ q[b, t, h // grp].astype(np.float64))
                np.testing.assert_allclose(o[b, t, h], ref, rtol=1e-12, atol=1e-15)


def test_p4_unit_gate_zero_beta_is_readout():
    q, k, v, g, beta, S0 = rand_inputs(4, T=7, state=True)
    g[:] = 0.0
    beta[:] = 0.0
    o, S = orc.seq(q, k, v, g, beta, S0)
    np.testing.assert_array_equal(S, S0)
    for t in range(7):
        for h in range(2):
            np.testing.assert_allclose(o[0, t, h], S0[0, h] @ q[0, t, 0].astype(np.float64),
                                       rtol=1e-13)


# --- P5: single token from a zero state ------------------------------------------------------

def test_p5_single_token_closed_form():
    q, k, v, g, beta, _ = rand_inputs(6, T=1, B=3)
    o, S = orc.seq(q, k, v, g, beta)
    for b in range(3):
        for h in range(2):
            kd, qd, vd = (x.astype(np.float64) for x in (k[b, 0, 0], q[b, 0, 0], v[b, 0, h]))
            bt = float(beta[b, 0, h])
            np.testing.assert_allclose(S[b, h], bt * np.outer(vd, kd), rtol=1e-14)
            np.testing.assert_allclose(o[b, 0, h], bt * (kd @ qd) * vd, rtol=1e-13, atol=1e-16)


# --- gated linear attention: mutually orthogonal keys from a zero state ----------------------

def test_orthogonal_keys_reduce_to_gated_linear_attention():
    # With S_0 = 0 and orthonormal keys, S_{t-1} k_t = 0, so the delta correction vanishes and
    # o_t = sum_{s<=t} (prod_{s<r<=t} a_r) beta_s (k_s . q_t) v_s  (decayed linear attention).
    rng = np.random.default_rng(9)
    dk, dv, T = 10, 3, 7
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:, :T].T.reshape(1, T, 1, dk)
    q = rng.standard_normal((1, T, 1, dk))
    v = rng.standard_normal((1, T, 1, dv))
    g = -rng.random((1, T, 1)) * 2
    beta = rng.uniform(0.1, 0.9, (1, T, 1))
    o, _ = orc.seq_literal(q, k, v, g, beta)          # exact fp64 keys
    for t in range(T):
        ref = np.zeros(dv)
        for s in range(t + 1):
            decay = np.exp(np.sum(g[0, s + 1:t + 1, 0]))
            ref += decay * beta[0, s, 0] * (k[0, s, 0] @ q[0, t, 0]) * v[0, s, 0]
        np.testing.assert_allclose(o[0, t, 0], ref, rtol=1e-11, atol=1e-13)
    # the C scan agrees on fp32-representable versions of the same inputs
    f = lambda x: x.astype(np.float32)  # noqa: E731
    o1, s1 = orc.seq(f(q), f(k), f(v), f(g), f(beta))
    o2, s2 = orc.seq_literal(f(q), f(k), f(v), f(g), f(beta))
    assert rel(o1, o2) < 1e-13 and rel(s1, s2) < 1e-13


# --- the state as an unrolled product ---------------------------------------------------------

def test_state_equals_unrolled_product_form():
    # S_T = S_0 M_1...M_T + sum_t beta_t v_t k_t^T M_{t+1}...M_T,  M_t = a_t (I - beta_t k_t k_t^T)
    q, k, v, g, beta, S0 = rand_inputs(11, T=8, state=True, dk=5, dv=3)
    _, S = orc.seq(q, k, v, g, beta, S0)
    kd, vd, bd = k.astype(np.float64), v.astype(np.float64), beta.astype(np.float64)
    a = np.exp(g.astype(np.float64))
    for h in range(2):
        Ms = [a[0, t, h] * (np.eye(5) - bd[0, t, h] * np.outer(kd[0, t, 0], kd[0, t, 0]))
              for t in range(8)]
        tail = [np.eye(5)] * 9                            # tail[t] = M_t ... M_{T-1} (0-based)
        for t in range(7, -1, -1):
            tail[t] = Ms[t] @ tail[t + 1]
        ref = S0[0, h] @ tail[0]
        for t in range(8):
            ref = ref + bd[0, t, h] * np.outer(vd[0, t, h], kd[0, t, 0]) @ tail[t + 1]
        np.testing.assert_allclose(S[0, h], ref, rtol=1e-12, atol=1e-14)


# --- P6: blockwise form against the token scan ------------------------------------------------

@pytest.mark.parametrize("chunk", [1, 3, 16, 37, 50])
def test_p6_chunked_matches_sequential(chunk):
    q, k, v, g, beta, S0 = rand_inputs(12, B=2, T=37, state=True, dk=6, dv=5)
    o1, s1 = orc.seq(q, k, v, g, beta, S0)
    o2, s2 = orc.chunked(q, k, v, g, beta, S0, chunk=chunk)
    assert rel(o2, o1) < 1e-12 and rel(s2, s1) < 1e-12


def test_p6_chunked_strong_decay_no_overflow():
    # Chunk-wide log-gate sums far below -88 (exp underflows in fp32): the blockwise form only
    # ever takes exp of gamma_r - gamma_s with s <= r, so it stays finite and exact.
    q, k, v, g, beta, S0 = rand_inputs(13, T=40, state=True, g_scale=12.0)
    o1, s1 = orc.seq(q, k, v, g, beta, S0)
    o2, s2 = orc.chunked(q, k, v, g, beta, S0, chunk=40)
    assert np.all(np.isfinite(o2)) and rel(o2, o1) < 1e-12 and rel(s2, s1) < 1e-12


# --- P7: affine in the starting state ---------------------------------------------------------

def test_p7_affine_in_initial_state():
    q, k, v, g, beta, S0 = rand_inputs(14, T=10, state=True)
    _, s_with = orc.seq(q, k, v, g, beta, S0)
    _, s_zero = orc.seq(q, k, v, g, beta, None)
    kd, bd = k.astype(np.float64), beta.astype(np.float64)
    a = np.exp(g.astype(np.float64))
    for h in range(2):
        M = np.eye(6)
        for t in range(10):
            M = M @ (a[0, t, h] * (np.eye(6) - bd[0, t, h] * np.outer(kd[0, t, 0], kd[0, t, 0])))
        np.testing.assert_allclose(s_with[0, h] - s_zero[0, h], S0[0, h] @ M, rtol=1e-11,
                                   atol=1e-13)


# --- P8/P9: segmenting and prefixes -----------------------------------------------------------

def test_p8_split_invariance_bitwise():
    q, k, v, g, beta, S0 = rand_inputs(15, B=2, T=30, state=True)
    o, s = orc.seq(q, k, v, g, beta, S0)
    for T1 in (1, 13, 29):
        oa, sa = orc.seq(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], S0)
        ob, sb = orc.seq(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], sa)
        np.testing.assert_array_equal(np.concatenate([oa, ob], axis=1), o)
        np.testing.assert_array_equal(sb, s)


def test_p9_prefix_causality_bitwise():
    q, k, v, g, beta, _ = rand_inputs(16, T=25)
    o, _ = orc.seq(q, k, v, g, beta)
    for Tp in (1, 8, 24):
        op, _ = orc.seq(q[:, :Tp], k[:, :Tp], v[:, :Tp], g[:, :Tp], beta[:, :Tp])
        np.testing.assert_array_equal(op, o[:, :Tp])


# --- P10: shared vs duplicated key heads ------------------------------------------------------

def test_p10_shared_heads_equal_duplicated_heads():
    q, k, v, g, beta, S0 = rand_inputs(17, T=9, Hk=2, Hv=4, state=True)
    o1, s1 = orc.seq(q, k, v, g, beta, S0)
    q2, k2 = np.repeat(q, 2, axis=2), np.repeat(k, 2, axis=2)   # head h reads q/k head h//2
    o2, s2 = orc.seq(q2, k2, v, g, beta, S0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


# --- P11: contraction bound --------------------------------------------------------------------

def test_p11_state_norm_bound():
    q, k, v, g, beta, S0 = rand_inputs(18, T=60, state=True, g_scale=0.2, beta_range=(0.0, 1.0))
    kd = k.astype(np.float64)
    kd /= np.linalg.norm(kd, axis=-1, keepdims=True)
    S = S0[0, 0].copy()
    for t in range(60):
        prev = np.linalg.norm(S, 2)
        _, Sn = orc.seq_literal(q[:, t:t + 1], kd[:, t:t + 1], v[:, t:t + 1], g[:, t:t + 1],
                                beta[:, t:t + 1], S[None, None].repeat(2, 1))
        S = Sn[0, 0]
        bound = np.exp(g[0, t, 0]) * prev + beta[0, t, 0] * np.linalg.norm(v[0, t, 0])
        assert np.linalg.norm(S, 2) <= bound * (1 + 1e-12)


# --- P12: fp32 twin against fp64 ----------------------------------------------------------------

def test_p12_fp32_scan_drift_is_small():
    q, k, v, g, beta, _ = rand_inputs(19, T=64, Hk=2, Hv=2, dk=32, dv=32)
    o64, s64 = orc.seq(q, k, v, g, beta)
    o32, s32 = orc.seq_f32(q, k, v, g, beta)
    assert rel(o32, o64) < 1e-5 and rel(s32, s64) < 1e-5


# --- selected (b, h) pairs are the same recurrences ---------------------------------------------

def test_pair_selection_matches_full_run():
    q, k, v, g, beta, S0 = rand_inputs(20, B=2, T=10, Hk=2, Hv=4, state=True)
    o, s = orc.seq(q, k, v, g, beta, S0)
    osel, ssel = orc.seq(q, k, v, g, beta, S0, pairs=[(1, 3), (0, 1)], rows_per_item=1)
    np.testing.assert_array_equal(osel[0], o[1, :, 3])
    np.testing.assert_array_equal(ssel[1], s[0, 1])


def test_decode_step_is_one_token_of_the_scan():
    q, k, v, g, beta, S0 = rand_inputs(21, B=2, T=1, Hk=2, Hv=4, state=True)
    o, s = orc.decode_step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], S0)
    o2, s2 = orc.seq_literal(q, k, v, g, beta, S0)
    assert rel(o, o2[:, 0]) < 1e-13 and rel(s, s2) < 1e-13


# --- P13: fused query/key L2 normalisation (qk_norm) -----------------------------------------
# Read of section "Reduce intermediate and state traffic" (the query/key preparation fused
# into the update): q_t, k_t -> x / sqrt(|x|^2 + 1e-6) before the recurrence.

def _pow2_scaled(x, rng, lo=0, hi=5):
    """x with each token's vector multiplied by a random power of two (exact in fp32)."""
    e = rng.integers(lo, hi, size=x.shape[:-1] + (1,))
    return (x * np.exp2(e)).astype(np.float32)


def test_p13_qknorm_write_then_read_raw_keys():
    # beta = 1 and q_t = k_t of any length: after normalisation |k^_t| = 1 - O(eps / |k|^2),
    # so o_t = S_t k^_t = v_t whatever a_t and S_{t-1} are.  Unnormalised keys of length
    # 1..16 would return up to 256 v_t, so a missing q or k normalisation fails here.
    rng = np.random.default_rng(31)
    q, k, v, g, beta, S0 = rand_inputs(31, B=2, T=10, Hk=1, Hv=2, state=True, g_scale=2.0)
    kr = _pow2_scaled(k, rng)
    beta[:] = 1.0
    o, _ = orc.seq(kr, kr, v, g, beta, S0, qk_norm=True)
    np.testing.assert_allclose(o, v.astype(np.float64), atol=5e-6)
    od, _ = orc.decode_step(kr[:, 3], kr[:, 3], v[:, 3], g[:, 3], beta[:, 3], S0, qk_norm=True)
    np.testing.assert_allclose(od, v[:, 3].astype(np.float64), atol=5e-6)


def test_p13_qknorm_scale_invariance():
    # positive per-token rescaling of q and k does not change the result (to eps / |x|^2)
    rng = np.random.default_rng(32)
    q, k, v, g, beta, S0 = rand_inputs(32, B=1, T=14, Hk=2, Hv=4, unit=False, state=True)
    o1, s1 = orc.seq(q, k, v, g, beta, S0, qk_norm=True)
    o2, s2 = orc.seq(_pow2_scaled(q, rng, -2, 4), _pow2_scaled(k, rng, -2, 4), v, g, beta, S0,
                     qk_norm=True)
    assert rel(o2, o1) < 1e-5 and rel(s2, s1) < 1e-5
    # and unit-length inputs are left (almost) unchanged
    qu, ku, *_ = rand_inputs(33, B=1, T=14, Hk=2, Hv=4, unit=True)
    o3, s3 = orc.seq(qu, ku, v, g, beta, S0, qk_norm=True)
    o4, s4 = orc.seq(qu, ku, v, g, beta, S0)
    assert rel(o3, o4) < 1e-5 and rel(s3, s4) < 1e-5


def test_p13_qknorm_zero_vectors_stay_finite():
    # k_t = 0 leaves only the decay (S_t = a_t S_{t-1}); q_t = 0 reads o_t = 0
    q, k, v, g, beta, S0 = rand_inputs(34, B=1, T=5, state=True, unit=False)
    q[:, 2] = 0.0
    k[:, 2] = 0.0
    o, s = orc.seq(q[:, :3], k[:, :3], v[:, :3], g[:, :3], beta[:, :3], S0, qk_norm=True)
    _, s2 = orc.seq(q[:, :2], k[:, :2], v[:, :2], g[:, :2], beta[:, :2], S0, qk_norm=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    np.testing.assert_array_equal(o[:, 2], 0.0)
    a = np.exp(g[0, 2].astype(np.float64))
    np.testing.assert_allclose(s[0], a[:, None, None] * s2[0], rtol=1e-14, atol=1e-300)
