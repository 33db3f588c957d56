"""Python binding of libgdn.so (include/gdn.h), via ctypes.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their data pointers and the current HIP stream are handed to the C
entry points of the same names, and a nonzero status raises ``GdnError``.  Every
step of the computation runs in the library's HIP kernels; there is no fallback.
PyTorch provides device memory and streams.
"""
import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_BF16 = 0
GDN_F32 = 1
_STATUS = {0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_SHAPE", 3: "GDN_ERR_UNSUPPORTED",
           4: "GDN_ERR_ALIGN", 5: "GDN_ERR_ALIAS", 6: "GDN_ERR_WORKSPACE", 7: "GDN_ERR_HIP"}
EXPORTS = ("gdn_prefill_workspace_bytes", "gdn_prefill", "gdn_prefill_qknorm", "gdn_prefill_ex",
           "gdn_prefill_sequential_max_tokens", "gdn_prefill_prepare", "gdn_prefill_scan",
           "gdn_decode_step", "gdn_decode_step_qknorm", "gdn_status_string", "gdn_abi_version",
           "gdn_prefill_noalloc", "gdn_decode_step_layers")
NOALLOC_SCRATCH_BYTES = 64 << 20   # GDN_NOALLOC_SCRATCH_BYTES

# flags of gdn_prefill_ex
GDN_QK_NORM = 1
GDN_PATH_SEQUENTIAL = 2
GDN_PATH_AUTO = 4
PATHS = {"blockwise": 0, "sequential": GDN_PATH_SEQUENTIAL, "auto": GDN_PATH_AUTO}


class DecodeLayer(ctypes.Structure):
    """gdn_decode_layer: one layer's device pointers for gdn_decode_step_layers."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("q", "k", "v", "g", "beta", "state_in",
                                               "state_out", "o")]


class GdnError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn}: {_STATUS.get(code, code)} ({gdn_status_string(code)})")


_lib = None


def lib():
    """The loaded library; raises if it has not been built (no fallback path exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.gdn_prefill_workspace_bytes.argtypes = [I] * 8
        L.gdn_prefill_workspace_bytes.restype = Z
        for fn in ("gdn_prefill", "gdn_prefill_qknorm", "gdn_prefill_prepare", "gdn_prefill_scan"):
            getattr(L, fn).argtypes = [P] * 8 + [I] * 8 + [P, Z, P]
            getattr(L, fn).restype = I
        for fn in ("gdn_decode_step", "gdn_decode_step_qknorm"):
            getattr(L, fn).argtypes = [P] * 8 + [I] * 6 + [P]
            getattr(L, fn).restype = I
        L.gdn_decode_step_layers.argtypes = [P, I, I, I, I, I, I, I, ctypes.c_uint, P]
        L.gdn_decode_step_layers.restype = I
        L.gdn_prefill_noalloc.argtypes = [P] * 8 + [I] * 8 + [P]
        L.gdn_prefill_noalloc.restype = I
        L.gdn_prefill_ex.argtypes = [P] * 8 + [I] * 8 + [P, Z, P, ctypes.c_uint]
        L.gdn_prefill_ex.restype = I
        L.gdn_prefill_sequential_max_tokens.argtypes = [I] * 6
        L.gdn_prefill_sequential_max_tokens.restype = I
        L.gdn_status_string.argtypes = [I]
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_abi_version.argtypes = []
        L.gdn_abi_version.restype = I
        _lib = L
    return _lib


def gdn_status_string(code: int) -> str:
    return lib().gdn_status_string(int(code)).decode()


def gdn_abi_version() -> int:
    return lib().gdn_abi_version()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"q/k/v/o must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError("tensors must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _f32(t, name):
    if t is not None and t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def gdn_prefill_workspace_bytes(B, T, Hk, Hv, dk, dv, chunk, dtype) -> int:
    if isinstance(dtype, torch.dtype):
        dtype = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    return int(lib().gdn_prefill_workspace_bytes(B, T, Hk, Hv, dk, dv, chunk, dtype))


def gdn_prefill(q, k, v, g, beta, state_in, o, state_out, chunk, workspace, stream=None):
    """Calls gdn_prefill.  q, k [B,T,Hk,dk]; v, o [B,T,Hv,dv] (bf16 or fp32); g, beta
    [B,T,Hv] fp32; state_in (or None) / state_out [B,Hv,dv,dk] fp32; workspace: a
    device tensor of at least gdn_prefill_workspace_bytes bytes (or None when T == 0)."""
    _prefill_call("gdn_prefill", q, k, v, g, beta, state_in, o, state_out, chunk, workspace,
                  stream)


def gdn_prefill_qknorm(q, k, v, g, beta, state_in, o, state_out, chunk, workspace, stream=None):
    """Calls gdn_prefill_qknorm (q and k L2-normalised inside); arguments as gdn_prefill."""
    _prefill_call("gdn_prefill_qknorm", q, k, v, g, beta, state_in, o, state_out, chunk,
                  workspace, stream)


def gdn_prefill_ex(q, k, v, g, beta, state_in, o, state_out, chunk, workspace, flags, stream=None):
    """Calls gdn_prefill_ex (flags: GDN_QK_NORM | GDN_PATH_SEQUENTIAL or GDN_PATH_AUTO);
    arguments as gdn_prefill, the workspace may be None on the sequential path."""
    _prefill_call("gdn_prefill_ex", q, k, v, g, beta, state_in, o, state_out, chunk, workspace,
                  stream, (int(flags),))


def gdn_prefill_noalloc(q, k, v, g, beta, state_in, o, state_out, chunk, stream=None):
    """Calls gdn_prefill_noalloc: gdn_prefill with the library's fixed device array as the
    workspace (nothing allocated); arguments as gdn_prefill without the workspace."""
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dt = _dt(q)
    for t in (k, v, o):
        if _dt(t) != dt:
            raise TypeError("q, k, v and o must share one dtype")
    for t, nm in ((g, "g"), (beta, "beta"), (state_in, "state_in"), (state_out, "state_out")):
        _f32(t, nm)
    rc = lib().gdn_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in),
                                   _ptr(o), _ptr(state_out), B, T, Hk, Hv, dk, dv, int(chunk), dt,
                                   _stream(stream))
    if rc != 0:
        raise GdnError("gdn_prefill_noalloc", rc)


def gdn_prefill_sequential_max_tokens(B, Hk, Hv, dk, dv, dtype) -> int:
    if isinstance(dtype, torch.dtype):
        dtype = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    return int(lib().gdn_prefill_sequential_max_tokens(B, Hk, Hv, dk, dv, dtype))


def gdn_prefill_prepare(q, k, v, g, beta, state_in, o, state_out, chunk, workspace, stream=None):
    """Calls gdn_prefill_prepare (the state-independent stage); arguments as gdn_prefill."""
    _prefill_call("gdn_prefill_prepare", q, k, v, g, beta, state_in, o, state_out, chunk,
                  workspace, stream)


def gdn_prefill_scan(q, k, v, g, beta, state_in, o, state_out, chunk, workspace, stream=None):
    """Calls gdn_prefill_scan (the chunk-to-chunk stage); arguments as gdn_prefill."""
    _prefill_call("gdn_prefill_scan", q, k, v, g, beta, state_in, o, state_out, chunk, workspace,
                  stream)


def _prefill_call(fn, q, k, v, g, beta, state_in, o, state_out, chunk, workspace, stream,
                  extra=()):
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dt = _dt(q)
    for t in (k, v, o):
        if _dt(t) != dt:
            raise TypeError("q, k, v and o must share one dtype")
    for t, nm in ((g, "g"), (beta, "beta"), (state_in, "state_in"), (state_out, "state_out")):
        _f32(t, nm)
    if tuple(k.shape) != (B, T, Hk, dk) or tuple(v.shape) != (B, T, Hv, dv) or \
            tuple(o.shape) != (B, T, Hv, dv) or tuple(g.shape) != (B, T, Hv) or \
            tuple(beta.shape) != (B, T, Hv) or tuple(state_out.shape) != (B, Hv, dv, dk) or \
            (state_in is not None and tuple(state_in.shape) != (B, Hv, dv, dk)):
        raise ValueError("inconsistent shapes")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = getattr(lib(), fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in),
                            _ptr(o), _ptr(state_out), B, T, Hk, Hv, dk, dv, int(chunk), dt,
                            _ptr(workspace), ws_bytes, _stream(stream), *extra)
    if rc != 0:
        raise GdnError(fn, rc)


def gdn_decode_step(q, k, v, g, beta, state_in, state_out, o, stream=None):
    """Calls gdn_decode_step.  q, k [B,Hk,dk]; v, o [B,Hv,dv]; g, beta [B,Hv] fp32;
    state_in / state_out [B,Hv,dv,dk] fp32 (may be the same tensor)."""
    _decode_call("gdn_decode_step", q, k, v, g, beta, state_in, state_out, o, stream)


def gdn_decode_step_qknorm(q, k, v, g, beta, state_in, state_out, o, stream=None):
    """Calls gdn_decode_step_qknorm (q and k L2-normalised inside); arguments as
    gdn_decode_step."""
    _decode_call("gdn_decode_step_qknorm", q, k, v, g, beta, state_in, state_out, o, stream)


def _decode_call(fn, q, k, v, g, beta, state_in, state_out, o, stream):
    B, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    dt = _dt(q)
    for t in (k, v, o):
        if _dt(t) != dt:
            raise TypeError("q, k, v and o must share one dtype")
    for t, nm in ((g, "g"), (beta, "beta"), (state_in, "state_in"), (state_out, "state_out")):
        _f32(t, nm)
    if tuple(k.shape) != (B, Hk, dk) or tuple(o.shape) != (B, Hv, dv) or \
            tuple(g.shape) != (B, Hv) or tuple(beta.shape) != (B, Hv) or \
            tuple(state_in.shape) != (B, Hv, dv, dk) or tuple(state_out.shape) != (B, Hv, dv, dk):
        raise ValueError("inconsistent shapes")
    rc = getattr(lib(), fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in),
                            _ptr(state_out), _ptr(o), B, Hk, Hv, dk, dv, dt, _stream(stream))
    if rc != 0:
        raise GdnError(fn, rc)


def gdn_decode_step_layers(layers, qk_norm=False, stream=None):
    """Calls gdn_decode_step_layers: one decode token through independent layers in one launch
    (per 32 layers).  ``layers``: a list of (q, k, v, g, beta, state_in, state_out, o) tensor
    tuples, each as for gdn_decode_step, all with the same sizes and dtype."""
    if not layers:
        raise ValueError("no layers")
    q0, v0 = layers[0][0], layers[0][2]
    B, Hk, dk = q0.shape
    Hv, dv = v0.shape[1], v0.shape[2]
    dt = _dt(q0)
    table = (DecodeLayer * len(layers))()
    for i, (q, k, v, g, beta, si, so, o) in enumerate(layers):
        for t in (k, v, o):
            if _dt(t) != dt:
                raise TypeError("q, k, v and o must share one dtype")
        for t, nm in ((g, "g"), (beta, "beta"), (si, "state_in"), (so, "state_out")):
            _f32(t, nm)
        if tuple(q.shape) != (B, Hk, dk) or tuple(k.shape) != (B, Hk, dk) or \
                tuple(v.shape) != (B, Hv, dv) or tuple(o.shape) != (B, Hv, dv) or \
                tuple(g.shape) != (B, Hv) or tuple(beta.shape) != (B, Hv) or \
                tuple(si.shape) != (B, Hv, dv, dk) or tuple(so.shape) != (B, Hv, dv, dk):
            raise ValueError(f"layer {i}: inconsistent shapes")
        table[i] = DecodeLayer(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(si), _ptr(so),
                               _ptr(o))
    rc = lib().gdn_decode_step_layers(table, len(layers), B, Hk, Hv, dk, dv, dt,
                                      GDN_QK_NORM if qk_norm else 0, _stream(stream))
    if rc != 0:
        raise GdnError("gdn_decode_step_layers", rc)


# -- conveniences that allocate outputs with torch --------------------------------------------

def _alloc_ctx(stream):
    """Allocation context of the stream the kernels are enqueued on.  torch's caching allocator
    ties a block to the stream it was allocated on: a workspace freed on return is then reused
    only by later work on that same stream (ordered after our kernels), never by another
    stream while our kernels may still read it."""
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream))
    return torch.cuda.stream(stream)


def prefill(q, k, v, g, beta, state=None, chunk=64, workspace=None, stream=None, qk_norm=False,
            path="blockwise"):
    """Returns (o, state_out); allocates o, state_out and (if needed and not given) the
    workspace.  qk_norm: L2-normalise q and k inside the kernels.  path: "blockwise"
    (gdn_prefill / gdn_prefill_qknorm), "sequential" or "auto" (gdn_prefill_ex)."""
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    flags = PATHS[path] | (GDN_QK_NORM if qk_norm else 0)
    seq = path == "sequential" or (
        path == "auto" and T <= gdn_prefill_sequential_max_tokens(B, Hk, Hv, dk, dv, q.dtype))
    with _alloc_ctx(stream):
        o = torch.empty((B, T, Hv, dv), dtype=q.dtype, device=q.device)
        s_out = torch.empty((B, Hv, dv, dk), dtype=torch.float32, device=q.device)
        if workspace is None and T > 0 and not seq:
            nb = gdn_prefill_workspace_bytes(B, T, Hk, Hv, dk, dv, chunk, q.dtype)
            workspace = torch.empty(nb, dtype=torch.uint8, device=q.device)
    if path == "blockwise":
        (gdn_prefill_qknorm if qk_norm else gdn_prefill)(q, k, v, g, beta, state, o, s_out, chunk,
                                                         workspace, stream)
    else:
        gdn_prefill_ex(q, k, v, g, beta, state, o, s_out, chunk, workspace, flags, stream)
    return o, s_out


def decode_step(q, k, v, g, beta, state, stream=None, qk_norm=False):
    """Updates ``state`` in place and returns o [B,Hv,dv].  qk_norm: L2-normalise q and k
    inside the kernel (gdn_decode_step_qknorm)."""
    with _alloc_ctx(stream):
        o = torch.empty(v.shape, dtype=q.dtype, device=q.device)
    (gdn_decode_step_qknorm if qk_norm else gdn_decode_step)(q, k, v, g, beta, state, state, o,
                                                             stream)
    return o
