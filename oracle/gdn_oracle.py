"""CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It shares no code with the GPU library (no kernels, headers,
helpers, tables or pre/post-processing) and never imports it.

Source of the method: the pages "Optimizing on-device inference for Apple
Silicon", section "Qwen creates three distinct workload shapes", describe the
Gated DeltaNet state: a learned gate keeps part of the old state, a delta update
writes in the current token, each token depends on the previous state, and the
same computation can be evaluated either by scanning tokens one at a time or
blockwise.  Section "Keep the recurrent state on chip" fixes the state and the
gate in fp32 (the oracle uses fp64) and the query/key activations in bf16.
Section "Bound temporary memory with prompt chunking" states that splitting a
prompt into segments that carry the recurrent state does not change the output.

The recurrence, per batch b and value head h (query/key head h // (Hv // Hk)),
state S of shape (dv, dk):

    a_t = exp(g_t)
    S_t = a_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
    o_t = S_t q_t

Functions
---------
seq_literal   the recurrence exactly as written above, with explicit dk x dk
              matrices (tiny inputs only).
seq           the C fp64 scan (rank-1 form), threaded over (b, h, rows).
seq_f32       the C fp32 twin (yardstick for rounding drift only).
chunked       the blockwise evaluation: per chunk, the decay-masked key Gram
              matrix, the unit-triangular inverse (I + A)^-1, the W and U~
              blocks, then the chunk-to-chunk state hand-off -- in fp64, one
              dense step at a time, to check the chunk algebra the GPU uses.
decode_step   one token of the recurrence (the T = 1 scan) on a given state.

seq and decode_step take qk_norm=True for the fused query/key preparation of
section "Reduce intermediate and state traffic", read as per-head L2
normalisation of q_t and k_t, x / sqrt(|x|^2 + 1e-6), done in fp64 first.

Every input array is widened exactly to float64 before use.  Layouts: q, k
[B,T,Hk,dk]; v [B,T,Hv,dv]; g, beta [B,T,Hv]; state [B,Hv,dv,dk]; o [B,T,Hv,dv].

Parity status: every function here is pinned by tests/test_oracle_pins.py
(closed forms, special cases, exact rational arithmetic, brute force); none is
"parity unpinned".
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(HERE, "libgdn_oracle.so")
        if not os.path.exists(path):
            from . import build as _b  # noqa: WPS433 (lazy: build only when absent)
            _b.build_oracle()
        lib = ctypes.CDLL(path)
        for name in ("gdn_oracle_seq_f64", "gdn_oracle_seq_f64_qknorm", "gdn_oracle_seq_f32"):
            fn = getattr(lib, name)
            P = ctypes.c_void_p
            fn.argtypes = [P, P, P, P, P, P, P, ctypes.c_int, P, P] + [ctypes.c_int] * 8
            fn.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _f32c(x):
    """fp32 C-contiguous copy; refuses values fp32 cannot hold exactly."""
    a = np.asarray(x)
    b = np.ascontiguousarray(a, dtype=np.float32)
    if a.dtype != np.float32 and a.dtype.kind == "f" and a.dtype.itemsize > 4:
        if not np.array_equal(b.astype(a.dtype), a):
            raise ValueError("oracle.seq takes values exactly representable in fp32")
    return b


def _dims(q, k, v, g, beta):
    B, T, Hk, dk = q.shape
    assert k.shape == (B, T, Hk, dk), (k.shape, q.shape)
    Bv, Tv, Hv, dv = v.shape
    assert (Bv, Tv) == (B, T)
    assert g.shape == (B, T, Hv) and beta.shape == (B, T, Hv)
    assert Hv % Hk == 0
    return B, T, Hk, Hv, dk, dv


def _run_c(fname, out_dtype, q, k, v, g, beta, state_in, pairs, nthreads, rows_per_item):
    B, T, Hk, Hv, dk, dv = _dims(q, k, v, g, beta)
    q, k, v, g, beta = (_f32c(x) for x in (q, k, v, g, beta))
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(Hv)]
    sel = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    n = sel.shape[0]
    o = np.zeros((n, T, dv), dtype=out_dtype)
    s = np.zeros((n, dv, dk), dtype=out_dtype)
    if state_in is not None:
        s_in = np.ascontiguousarray(np.asarray(state_in, dtype=np.float64))
        assert s_in.shape == (B, Hv, dv, dk)
        s_ptr = s_in.ctypes.data
    else:
        s_in, s_ptr = None, None
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    rc = getattr(_lib(), fname)(q.ctypes.data, k.ctypes.data, v.ctypes.data, g.ctypes.data,
                                beta.ctypes.data, s_ptr, sel.ctypes.data, n, o.ctypes.data,
                                s.ctypes.data, B, T, Hk, Hv, dk, dv, int(nthreads),
                                int(rows_per_item))
    if rc != 0:
        raise ValueError(f"{fname} rejected its arguments (code {rc})")
    del s_in
    return sel, o, s


def seq(q, k, v, g, beta, state_in=None, pairs=None, nthreads=None, rows_per_item=16,
        qk_norm=False):
    """fp64 sequential scan (C).  Returns (o [B,T,Hv,dv], state [B,Hv,dv,dk]) when
    ``pairs`` is None, else (o_sel [n,T,dv], s_sel [n,dv,dk]) for the listed
    (b, h) pairs only -- each pair is an independent recurrence.  qk_norm: every
    q_t and k_t is first replaced by x / sqrt(|x|^2 + 1e-6) in fp64."""
    fname = "gdn_oracle_seq_f64_qknorm" if qk_norm else "gdn_oracle_seq_f64"
    sel, o, s = _run_c(fname, np.float64, q, k, v, g, beta, state_in, pairs, nthreads,
                       rows_per_item)
    if pairs is not None:
        return o, s
    B, T, _, Hv, dk, dv = _dims(q, k, v, g, beta)
    return (o.reshape(B, Hv, T, dv).transpose(0, 2, 1, 3).copy(), s.reshape(B, Hv, dv, dk))


def seq_f32(q, k, v, g, beta, state_in=None, pairs=None, nthreads=None, rows_per_item=16):
    """The same scan carried out in fp32 (C); same return convention as ``seq``."""
    sel, o, s = _run_c("gdn_oracle_seq_f32", np.float32, q, k, v, g, beta, state_in, pairs,
                       nthreads, rows_per_item)
    if pairs is not None:
        return o, s
    B, T, _, Hv, dk, dv = _dims(q, k, v, g, beta)
    return (o.reshape(B, Hv, T, dv).transpose(0, 2, 1, 3).copy(), s.reshape(B, Hv, dv, dk))


def seq_literal(q, k, v, g, beta, state_in=None):
    """The recurrence with explicit matrices, in fp64, one token at a time:
    S <- exp(g) * S @ (I - beta k k^T) + beta v k^T ;  o = S q."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    B, T, Hk, Hv, dk, dv = _dims(q, k, v, g, beta)
    grp = Hv // Hk
    o = np.zeros((B, T, Hv, dv))
    S_all = np.zeros((B, Hv, dv, dk))
    eye = np.eye(dk)
    for b in range(B):
        for h in range(Hv):
            hk = h // grp
            S = np.zeros((dv, dk)) if state_in is None else np.array(state_in[b, h], dtype=np.float64)
            for t in range(T):
                kt = k[b, t, hk]
                a = np.exp(g[b, t, h])
                bt = beta[b, t, h]
                S = a * S @ (eye - bt * np.outer(kt, kt)) + bt * np.outer(v[b, t, h], kt)
                o[b, t, h] = S @ q[b, t, hk]
            S_all[b, h] = S
    return o, S_all


def chunked(q, k, v, g, beta, state_in=None, chunk=16):
    """Blockwise evaluation of the same recurrence in fp64.

    The pages say the scan can be regrouped into blocks that expose matrix
    operations and token-level parallelism.  Unrolling the recurrence inside a
    chunk of n tokens that starts from state S0 (our derivation; the pages give
    the idea, not the algebra):

      gamma_r = g_1 + ... + g_r               (within-chunk log-gate prefix)
      A[r,s]  = beta_r exp(gamma_r - gamma_s) (k_r . k_s)   for s < r, else 0
      R       = (I + A)^-1                    (unit lower triangular)
      W       = R diag(beta exp(gamma)) K      Ut = R diag(beta) V
      U       = Ut - W S0^T                   (row r = the delta written at token r)
      O       = diag(exp(gamma)) Q S0^T + (M * Q K^T) U,   M[r,s] = exp(gamma_r-gamma_s), s <= r
      S_next  = exp(gamma_n) S0 + U^T diag(exp(gamma_n - gamma)) K

    R is formed with a dense solve; everything else is a plain matrix product.
    A final chunk shorter than ``chunk`` is handled with n < chunk.
    """
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    B, T, Hk, Hv, dk, dv = _dims(q, k, v, g, beta)
    grp = Hv // Hk
    o = np.zeros((B, T, Hv, dv))
    S_all = np.zeros((B, Hv, dv, dk))
    for b in range(B):
        for h in range(Hv):
            hk = h // grp
            S = np.zeros((dv, dk)) if state_in is None else np.array(state_in[b, h], dtype=np.float64)
            for c0 in range(0, T, chunk):
                c1 = min(T, c0 + chunk)
                n = c1 - c0
                K = k[b, c0:c1, hk]          # n x dk
                Q = q[b, c0:c1, hk]          # n x dk
                V = v[b, c0:c1, h]           # n x dv
                bt = beta[b, c0:c1, h]       # n
                gam = np.cumsum(g[b, c0:c1, h])
                D = gam[:, None] - gam[None, :]          # gamma_r - gamma_s
                low = np.tril(np.ones((n, n)), -1)       # s < r
                lowd = np.tril(np.ones((n, n)), 0)       # s <= r
                A = bt[:, None] * np.exp(np.where(low > 0, D, 0.0)) * (K @ K.T) * low
                R = np.linalg.solve(np.eye(n) + A, np.eye(n))
                W = R @ ((bt * np.exp(gam))[:, None] * K)
                Ut = R @ (bt[:, None] * V)
                U = Ut - W @ S.T
                M = np.exp(np.where(lowd > 0, D, 0.0)) * lowd
                o[b, c0:c1, h] = np.exp(gam)[:, None] * (Q @ S.T) + (M * (Q @ K.T)) @ U
                S = np.exp(gam[-1]) * S + U.T @ (np.exp(gam[-1] - gam)[:, None] * K)
            S_all[b, h] = S
    return o, S_all


def decode_step(q, k, v, g, beta, state, qk_norm=False):
    """One token of the recurrence (fp64, C scan) on the given state.

    q, k [B,Hk,dk]; v [B,Hv,dv]; g, beta [B,Hv]; state [B,Hv,dv,dk].
    Returns (o [B,Hv,dv], new_state [B,Hv,dv,dk])."""
    q, k, v, g, beta = (np.asarray(x)[:, None] for x in (q, k, v, g, beta))
    o, s = seq(q, k, v, g, beta, state_in=state, qk_norm=qk_norm)
    return o[:, 0], s
