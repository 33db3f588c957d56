"""CPU-only checks of the C-ABI library: it loads, exports every entry point that
include/gdn.h declares, reports its ABI version, sizes the workspace, and rejects
bad arguments synchronously -- before anything is enqueued -- with the documented
status codes.  No call here reaches a kernel launch (all arguments are invalid in
at least one way, and validation runs first), so no GPU is needed."""
import ctypes
import os
import re

import pytest

from linear_recurrent_attention_gated_amd import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = gdn.lib()
    declared = header_functions()
    assert set(declared) == set(gdn.EXPORTS), declared
    for name in declared:
        assert hasattr(L, name), name


def test_abi_version_and_status_strings():
    assert gdn.gdn_abi_version() == 1
    for code in range(8):
        assert gdn.gdn_status_string(code)
    assert gdn.gdn_status_string(99) == "unknown status"


def test_workspace_bytes():
    # prefill at T=4096, Hk=16, Hv=32, dk=dv=128, chunk 64, bf16:
    # k and q fragments: 16*4096*128*2 each; Z: 32 heads * 64 chunks * 128*64*2;
    # P': 32*4096*64*2; gate factors: 32 heads * 64 chunks * (2*64 + 4) floats
    expect = 2 * 16 * 4096 * 128 * 2 + 32 * 64 * 128 * 64 * 2 + 32 * 4096 * 64 * 2 + 32 * 64 * 132 * 4
    assert gdn.gdn_prefill_workspace_bytes(1, 4096, 16, 32, 128, 128, 64, 0) == expect
    assert gdn.gdn_prefill_workspace_bytes(1, 0, 16, 32, 128, 128, 64, 0) == 0
    assert gdn.gdn_prefill_workspace_bytes(1, 64, 16, 32, 96, 128, 64, 0) == 0     # unsupported
    # a ragged tail rounds up to whole chunks
    assert gdn.gdn_prefill_workspace_bytes(1, 65, 1, 1, 32, 32, 16, 1) == \
        gdn.gdn_prefill_workspace_bytes(1, 80, 1, 1, 32, 32, 16, 1)


# Fake, well-separated "device" addresses: never dereferenced, validation rejects first.
BASE = 1 << 40
MB = 1 << 20


def _prefill(fn="gdn_prefill", **kw):
    a = dict(q=BASE, k=BASE + 10 * MB, v=BASE + 20 * MB, g=BASE + 40 * MB, beta=BASE + 41 * MB,
             state_in=BASE + 50 * MB, o=BASE + 60 * MB, state_out=BASE + 80 * MB, B=1, T=64, Hk=2,
             Hv=4, dk=32, dv=32, chunk=16, dtype=0, ws=BASE + 100 * MB, ws_bytes=0, stream=None)
    a.update(kw)
    if "ws_bytes" not in kw:
        a["ws_bytes"] = gdn.gdn_prefill_workspace_bytes(a["B"], a["T"], a["Hk"], a["Hv"], a["dk"],
                                                        a["dv"], a["chunk"], a["dtype"])
    return getattr(gdn.lib(), fn)(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state_in"], a["o"],
                                 a["state_out"], a["B"], a["T"], a["Hk"], a["Hv"], a["dk"], a["dv"],
                                 a["chunk"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


def _decode(fn="gdn_decode_step", **kw):
    a = dict(q=BASE, k=BASE + MB, v=BASE + 2 * MB, g=BASE + 3 * MB, beta=BASE + 4 * MB,
             state_in=BASE + 10 * MB, state_out=BASE + 10 * MB, o=BASE + 30 * MB, B=1, Hk=2, Hv=4,
             dk=32, dv=32, dtype=0, stream=None)
    a.update(kw)
    return getattr(gdn.lib(), fn)(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state_in"],
                                  a["state_out"], a["o"], a["B"], a["Hk"], a["Hv"], a["dk"],
                                  a["dv"], a["dtype"], a["stream"])


# Each case breaks exactly one rule; the rest of the call is valid.
PREFILL_ERRORS = [
    (dict(q=None), 1), (dict(state_out=None), 1), (dict(beta=None), 1),
    (dict(Hv=3), 2), (dict(B=0), 2), (dict(T=-1), 2), (dict(Hk=0), 2),
    (dict(dk=48), 3), (dict(dv=256), 3), (dict(chunk=128), 3), (dict(chunk=8), 3), (dict(dtype=7), 3),
    (dict(q=BASE + 2), 4), (dict(o=BASE + 60 * MB + 8), 4), (dict(g=BASE + 40 * MB + 2), 4),
    (dict(state_in=BASE + 50 * MB + 4), 4),
    (dict(o=BASE + 10 * MB), 5),                         # o overlaps k
    (dict(state_out=BASE + 60 * MB + 4096), 5),          # state_out overlaps o
    (dict(state_out=BASE + 50 * MB + 4096), 5),          # partial overlap with state_in
    (dict(ws=BASE + 20 * MB), 5),                        # workspace overlaps v
    (dict(ws_bytes=1024), 6), (dict(ws=None), 6),
]


@pytest.mark.parametrize("fn", ["gdn_prefill", "gdn_prefill_qknorm", "gdn_prefill_prepare",
                                "gdn_prefill_scan"])
@pytest.mark.parametrize("kw,code", PREFILL_ERRORS)
def test_prefill_rejects(kw, code, fn):
    assert _prefill(fn=fn, **kw) == code


@pytest.mark.parametrize("kw,code", [c for c in PREFILL_ERRORS if not ({"ws", "ws_bytes"} & set(c[0]))]
                         + [(dict(B=64, T=64, Hk=16, Hv=32, dk=128, dv=128, chunk=64), 6)])
def test_prefill_noalloc_rejects(kw, code):
    # gdn_prefill_noalloc validates every argument before it looks up its device array (the
    # last case: one chunk's blocks, ~84 MB, exceed the 64 MiB array)
    a = dict(q=BASE, k=BASE + 10 * MB, v=BASE + 20 * MB, g=BASE + 40 * MB, beta=BASE + 41 * MB,
             state_in=BASE + 50 * MB, o=BASE + 60 * MB, state_out=BASE + 80 * MB, B=1, T=64, Hk=2,
             Hv=4, dk=32, dv=32, chunk=16, dtype=0)
    if "B" in kw:   # the large shape needs room between the fake buffers
        a.update(k=BASE + 200 * MB, v=BASE + 400 * MB, g=BASE + 600 * MB, beta=BASE + 610 * MB,
                 state_in=BASE + 700 * MB, o=BASE + 900 * MB, state_out=BASE + 1000 * MB)
    a.update(kw)
    rc = gdn.lib().gdn_prefill_noalloc(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state_in"],
                                       a["o"], a["state_out"], a["B"], a["T"], a["Hk"], a["Hv"],
                                       a["dk"], a["dv"], a["chunk"], a["dtype"], None)
    assert rc == code


@pytest.mark.parametrize("flags", [8, 2 | 4, 0x100])
def test_prefill_ex_rejects_flags(flags):
    L = gdn.lib()
    ws = gdn.gdn_prefill_workspace_bytes(1, 64, 2, 4, 32, 32, 16, 0)
    rc = L.gdn_prefill_ex(BASE, BASE + 10 * MB, BASE + 20 * MB, BASE + 40 * MB, BASE + 41 * MB,
                          BASE + 50 * MB, BASE + 60 * MB, BASE + 80 * MB, 1, 64, 2, 4, 32, 32, 16,
                          0, BASE + 100 * MB, ws, None, flags)
    assert rc == 3


@pytest.mark.parametrize("T", [64, 1])   # T = 1 from a given state: GDN_PATH_AUTO's decode step
@pytest.mark.parametrize("flags", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("kw,code", [(dict(q=None), 1), (dict(Hv=3), 2), (dict(dk=48), 3),
                                     (dict(q=BASE + 2), 4), (dict(o=BASE + 10 * MB), 5),
                                     (dict(ws=BASE + 60 * MB), 5)])
def test_prefill_ex_validates_on_every_path(kw, code, flags, T):
    # every path checks the same arguments, the workspace (even where it goes unused) included
    a = dict(q=BASE, o=BASE + 60 * MB, Hv=4, dk=32, ws=BASE + 100 * MB)
    a.update(kw)
    rc = gdn.lib().gdn_prefill_ex(a["q"], BASE + 10 * MB, BASE + 20 * MB, BASE + 40 * MB,
                                  BASE + 41 * MB, BASE + 50 * MB, a["o"], BASE + 80 * MB, 1, T,
                                  2, a["Hv"], a["dk"], 32, 16, 0, a["ws"], 1 << 26, None,
                                  flags)
    assert rc == code


def test_sequential_crossover_follows_the_measured_table():
    f = gdn.gdn_prefill_sequential_max_tokens
    # batch 1 at 32 value heads: the measured crossovers (bf16, fp32) x (d = 32, 64, 128)
    assert [f(1, 16, 32, d, d, 0) for d in (32, 64, 128)] == [43, 42, 42]
    assert [f(1, 16, 32, d, d, 1) for d in (32, 64, 128)] == [89, 96, 110]
    assert f(1, 2, 4, 128, 128, 0) == 42                   # fewer heads: unchanged
    assert 19 <= f(4, 16, 32, 128, 128, 0) <= 29           # batch 4 measured 24
    assert 41 <= f(4, 16, 32, 128, 128, 1) <= 51           # batch 4 measured 46
    assert 25 <= f(4, 16, 32, 64, 64, 0) <= 33             # 2,048 waves, measured 28
    assert 96 < f(1, 16, 32, 64, 128, 1) < 110             # between the tabulated sizes
    assert f(1000, 16, 32, 128, 128, 0) >= 1
    assert f(1, 16, 32, 96, 128, 0) == 0                   # unsupported size


DECODE_ERRORS = [
    (dict(state_in=None), 1), (dict(o=None), 1),
    (dict(Hv=5), 2), (dict(B=0), 2),
    (dict(dk=16), 3), (dict(dtype=2), 3),
    (dict(k=BASE + MB + 4), 4), (dict(state_out=BASE + 12 * MB + 8), 4),
    (dict(o=BASE + 2 * MB), 5),                          # o overlaps v
    (dict(state_out=BASE + 10 * MB + 1024), 5),          # partial state overlap
    (dict(state_out=BASE + 64), 5),                      # state_out overlaps q
]


@pytest.mark.parametrize("fn", ["gdn_decode_step", "gdn_decode_step_qknorm"])
@pytest.mark.parametrize("kw,code", DECODE_ERRORS)
def test_decode_rejects(kw, code, fn):
    assert _decode(fn=fn, **kw) == code


def _layers(n, **kw):
    # n layers of fake, well-separated buffers (64 MB apart); kw overrides fields of layer 1
    T = (gdn.DecodeLayer * n)()
    for i in range(n):
        b = BASE + i * 64 * MB
        T[i] = gdn.DecodeLayer(b, b + MB, b + 2 * MB, b + 3 * MB, b + 4 * MB, b + 10 * MB,
                               b + 10 * MB, b + 30 * MB)
    for f, val in kw.items():
        setattr(T[1], f, val)
    return T


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(o=None), 1),
    (dict(k=BASE + 64 * MB + MB + 4), 4),
    (dict(o=BASE + 64 * MB + 2 * MB), 5),                   # o overlaps its own v
    (dict(state_out=BASE + 10 * MB), 5),                     # writes layer 0's state
    (dict(o=BASE + 2 * MB), 5),                              # writes over layer 0's v
    (dict(state_in=BASE + 30 * MB, state_out=BASE + 64 * MB + 10 * MB), 5),   # reads layer 0's o
])
def test_decode_layers_rejects(kw, code):
    L = gdn.lib()
    assert L.gdn_decode_step_layers(_layers(3, **kw), 3, 1, 2, 4, 32, 32, 0, 0, None) == code


def test_decode_layers_rejects_bad_calls():
    L = gdn.lib()
    assert L.gdn_decode_step_layers(None, 3, 1, 2, 4, 32, 32, 0, 0, None) == 1
    assert L.gdn_decode_step_layers(_layers(3), 0, 1, 2, 4, 32, 32, 0, 0, None) == 2
    assert L.gdn_decode_step_layers(_layers(3), 3, 1, 2, 5, 32, 32, 0, 0, None) == 2
    assert L.gdn_decode_step_layers(_layers(3), 3, 1, 2, 4, 48, 32, 0, 0, None) == 3
    assert L.gdn_decode_step_layers(_layers(3), 3, 1, 2, 4, 32, 32, 0, 2, None) == 3


def test_python_binding_raises_with_status():
    with pytest.raises(gdn.GdnError) as ei:
        raise gdn.GdnError("gdn_prefill", 5)
    assert "GDN_ERR_ALIAS" in str(ei.value)
