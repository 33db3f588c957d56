"""GPU checks against closed forms that the recurrence itself fixes, at any size.

The recurrence S_t = a_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T, o_t = S_t q_t
("Optimizing on-device inference for Apple Silicon", section "Qwen creates three distinct
workload shapes": the gate retains the state, the delta update writes the current token) has
two cases with a plain answer:

* beta = 0: nothing is written.  The state only decays, S_T = exp(sum_t g_t) S_0, and every
  output reads the decayed start state, o_t = exp(sum_{s<=t} g_s) S_0 q_t.  Checked at the full
  4K prefill shape on every head and token.
* a = 1 (g = 0), beta = 1, distinct standard-basis keys (orthonormal, and exact in bf16) and
  q_t = k_t, from a zero state: each token writes v_t into an empty column pi(t) of the state,
  and reading it back returns v_t.  Every product the kernels form then has at most one nonzero
  term, so o_t = v_t and S_T[:, pi(t)] = v_t hold bit for bit in both builds, on every path
  (blockwise at each chunk size, token-sequential, automatic choice, repeated decode steps).
"""
import pytest
import torch
import torch.nn.functional as F

from linear_recurrent_attention_gated_amd import gdn
from tests.gpu_util import TOL_O, nrel, np32, say

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _no_write_inputs(B, T, Hk, Hv, dk, dv, dt, seed):
    gen = torch.Generator("cpu").manual_seed(seed)
    rn = lambda *s: torch.randn(*s, generator=gen)  # noqa: E731
    q = F.normalize(rn(B, T, Hk, dk), dim=-1).to(dt)
    k = F.normalize(rn(B, T, Hk, dk), dim=-1).to(dt)
    v = rn(B, T, Hv, dv).to(dt)
    # slow decay (a ~ 0.999), so that the state is still ~exp(-4) of its start after 4K tokens
    g = -F.softplus(rn(B, T, Hv) - 7.0)
    beta = torch.zeros(B, T, Hv)
    s0 = rn(B, Hv, dv, dk) * 0.1
    return q, k, v, g.contiguous(), beta, s0


def _no_write_expected(q, g, s0, Hv):
    """fp64 closed form: per (b, h), o_t = exp(G_t) S_0 q_t with G the running sum of g."""
    B, T, Hk, dk = q.shape
    G = torch.cumsum(g.double(), dim=1)                                   # [B, T, Hv]
    qv = q.double().repeat_interleave(Hv // Hk, dim=2)                    # [B, T, Hv, dk]
    o = torch.einsum("bhij,bthj->bthi", s0.double(), qv) * torch.exp(G)[..., None]
    s_t = s0.double() * torch.exp(G[:, -1])[:, :, None, None]
    return o.numpy(), s_t.numpy()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("path,T", [("blockwise", 4096), ("sequential", 512), ("auto", 40)])
def test_no_write_state_decays_by_the_gate_product(dt, path, T):
    B, Hk, Hv, dk, dv = 1, 16, 32, 128, 128
    q, k, v, g, beta, s0 = _no_write_inputs(B, T, Hk, Hv, dk, dv, DT[dt], seed=11)
    say("beta=0 decay", dt, path, (B, T, Hk, Hv, dk, dv))
    o, s = gdn.prefill(q.cuda(), k.cuda(), v.cuda(), g.cuda(), beta.cuda(), s0.cuda(), chunk=64,
                       path=path)
    torch.cuda.synchronize()
    o_ref, s_ref = _no_write_expected(q, g, s0, Hv)
    eo, es = nrel(np32(o), o_ref), nrel(s.cpu().numpy(), s_ref)
    say("beta=0 decay errors", dt, path, eo, es)
    # the state is only ever scaled by fp32 gate factors (blockwise once per chunk, token by
    # token in the sequential form): far inside its tolerance in both builds
    tol = 1e-5 if path == "blockwise" else 1e-4
    assert es < tol
    # o carries the bf16 rounding of the output (and, blockwise, of the state operand of Q S^T)
    assert eo < (1e-2 if dt == "bf16" else tol)
    assert eo < TOL_O


def _write_read_inputs(B, T, Hk, Hv, dk, dv, dt, seed):
    assert T <= dk
    gen = torch.Generator("cpu").manual_seed(seed)
    perm = torch.stack([torch.stack([torch.randperm(dk, generator=gen)[:T] for _ in range(Hk)])
                        for _ in range(B)])                                # [B, Hk, T]
    k = torch.zeros(B, T, Hk, dk)
    for b in range(B):
        for hk in range(Hk):
            k[b, torch.arange(T), hk, perm[b, hk]] = 1.0
    k = k.to(dt)
    v = torch.randn(B, T, Hv, dv, generator=gen).to(dt)
    g = torch.zeros(B, T, Hv)
    beta = torch.ones(B, T, Hv)
    s_ref = torch.zeros(B, Hv, dv, dk)
    for b in range(B):
        for h in range(Hv):
            s_ref[b, h][:, perm[b, h // (Hv // Hk)]] = v[b, :, h].float().t()
    return k, v, g, beta, s_ref


WRITE_READ = [
    # B, T, Hk, Hv, dk, dv
    (1, 128, 2, 4, 128, 128),
    (2, 100, 1, 2, 128, 32),
    (1, 64, 2, 2, 64, 128),
    (1, 32, 1, 2, 32, 32),
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", WRITE_READ, ids=[f"B{c[0]}T{c[1]}h{c[2]}-{c[3]}d{c[4]}x{c[5]}"
                                                  for c in WRITE_READ])
def test_orthonormal_write_then_read_is_exact(case, dt):
    B, T, Hk, Hv, dk, dv = case
    k, v, g, beta, s_ref = _write_read_inputs(B, T, Hk, Hv, dk, dv, DT[dt], seed=5)
    kd, vd, gd, bd = k.cuda(), v.cuda(), g.cuda(), beta.cuda()
    runs = [(f"blockwise c{c}", dict(chunk=c, path="blockwise")) for c in (16, 32, 64)]
    runs += [("sequential", dict(path="sequential")), ("auto", dict(path="auto"))]
    for name, kw in runs:
        say("write-read", dt, name, case)
        o, s = gdn.prefill(kd, kd, vd, gd, bd, None, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o.cpu(), v), name
        assert torch.equal(s.cpu(), s_ref), name
    # the same tokens one decode step at a time (state updated in place)
    say("write-read", dt, "decode steps", case)
    st = torch.zeros(B, Hv, dv, dk, device="cuda")
    for t in range(T):
        o = gdn.decode_step(kd[:, t].contiguous(), kd[:, t].contiguous(), vd[:, t].contiguous(),
                            gd[:, t].contiguous(), bd[:, t].contiguous(), st)
        torch.cuda.synchronize()
        assert torch.equal(o.cpu(), v[:, t]), t
    assert torch.equal(st.cpu(), s_ref)
