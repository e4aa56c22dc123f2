"""Python binding of liblmtopk: the LM-head projection fused with exact top-k on MI355X.

Argument marshalling only: tensors are checked and their device pointers,
sizes and the current HIP stream are handed to the C ABI declared in
include/lmtopk.h; every step of the computation runs in the library's HIP
kernels.  PyTorch supplies device memory and streams.

Entry points mirror the lm-head-topk page (section "Usage"):
    lm_head_topk_binary(act_q, act_scale, wq, wscale, bias=None, group_size=128, k=50, ...)
    lm_head_topk_dense(hidden, weight, k=50, bias=None, ...)
plus pack_binary (offline packing of a dense head) and topk_logits (the
selection stage alone, on logits already in memory).  Each returns
(values [M, k] float32, indices [M, k] int64), sorted by value descending,
ties to the lower vocabulary index; given `sampling=Sampling(...)` each also
draws one token per row from its k survivors (logits-processor page,
sections "API" and "Method") and returns (values, indices, tokens).
sample(logits, ...) is the page's sample() on logits in memory, restricted to
the top-k.

Importing this module raises ImportError if the built library is missing:
there is no fallback path.
"""

import ctypes
import functools
import os

import torch

__all__ = [
    "LmTopkError",
    "layout_version",
    "packed_bytes",
    "workspace_bytes",
    "binary_plan",
    "pack_binary",
    "lm_head_topk_binary",
    "lm_head_topk_dense",
    "topk_logits",
    "library_path",
    "new_workspace",
    "workspace_init",
    "Sampling",
    "sample",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# LMTOPK_LIBRARY names another build of the same library to load instead
# (for comparing builds); by default the in-tree build is loaded.
_LIB_PATH = os.environ.get("LMTOPK_LIBRARY") or os.path.join(_HERE, "_lib", "liblmtopk.so")

GROUP_SIZE = 128
MAX_ROWS = 8
MAX_K = 2048
_F32, _BF16 = 0, 1


class LmTopkError(ValueError):
    """A status other than LMTOPK_OK returned by the library."""

    def __init__(self, status, text):
        super().__init__(f"liblmtopk status {status}: {text}")
        self.status = status


class _SamplingC(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_k", ctypes.c_int32),
                ("top_p", ctypes.c_float), ("min_p", ctypes.c_float),
                ("temperature_rows", ctypes.c_void_p), ("top_k_rows", ctypes.c_void_p),
                ("top_p_rows", ctypes.c_void_p), ("min_p_rows", ctypes.c_void_p),
                ("seed", ctypes.c_uint64), ("offset", ctypes.c_uint64),
                ("offset_device", ctypes.c_void_p), ("tokens", ctypes.c_void_p),
                ("kept", ctypes.c_void_p)]


class _Options(ctypes.Structure):
    _fields_ = [("chunk_rows", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("score_events", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("allowed", ctypes.c_void_p), ("sampling", ctypes.POINTER(_SamplingC))]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"liblmtopk is not built ({_LIB_PATH} missing); run "
            "`python lm_head_projection_amd/build.py` (needs hipcc for gfx950)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    psz = ctypes.POINTER(ctypes.c_size_t)
    pi32 = ctypes.POINTER(ctypes.c_int32)
    popt = ctypes.POINTER(_Options)
    sig = {
        "lmtopk_layout_version": ([], i32),
        "lmtopk_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "lmtopk_packed_bytes": ([i64, i64, i32, psz, psz], ctypes.c_int),
        "lmtopk_workspace_bytes": ([i64, i64, i32, popt, psz], ctypes.c_int),
        "lmtopk_binary_plan": ([i64, i64, i64, i32, popt, pi32, pi32, pi32], ctypes.c_int),
        "lmtopk_workspace_init": ([vp, sz, vp], ctypes.c_int),
        "lmtopk_pack_binary": ([vp, ctypes.c_int, i64, i64, i32, vp, vp, vp], ctypes.c_int),
        "lmtopk_binary": ([vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, vp, vp, sz, popt, vp],
                          ctypes.c_int),
        "lmtopk_dense": ([vp, vp, ctypes.c_int, vp, i64, i64, i64, i32, vp, vp, vp, sz, popt, vp],
                         ctypes.c_int),
        "lmtopk_select": ([vp, i64, i64, i64, i32, vp, vp, vp, sz, popt, vp], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


_lib = _load()


def library_path():
    return _LIB_PATH


def _check(status):
    if status != 0:
        raise LmTopkError(status, _lib.lmtopk_status_string(status).decode())


def layout_version():
    return int(_lib.lmtopk_layout_version())


@functools.lru_cache(maxsize=256)
def packed_bytes(V, H, group_size=GROUP_SIZE):
    """(wq_bytes, wscale_bytes) of a packed V x H head."""
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(_lib.lmtopk_packed_bytes(V, H, group_size, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


class Sampling:
    """Parameters of the token draw over the top-k survivors (logits-processor
    page, section "API": sample(logits, temperature, top_k, top_p, min_p,
    seed, offset)).

    temperature, top_k, top_p, min_p: a Python number for every row, or a GPU
    tensor [M] per row (float32; top_k int32).  temperature <= 0 is greedy;
    top_k <= 0, top_p >= 1 and min_p <= 0 switch their filter off (the draw
    never leaves the call's k survivors; a scalar top_k above k is an error).
    seed: int.  offset: int, or a GPU tensor [1] (int64/uint64) read when the
    call runs, so that a captured graph can be replayed with a new offset.
    """

    def __init__(self, temperature=1.0, top_k=0, top_p=1.0, min_p=0.0, seed=0, offset=0):
        self.temperature, self.top_k, self.top_p, self.min_p = temperature, top_k, top_p, min_p
        self.seed, self.offset = int(seed), offset

    def _c(self, M, tokens, kept):
        c = _SamplingC()
        keep = []

        def split(name, value, dtype, conv):
            if isinstance(value, torch.Tensor):
                _need_cuda(name, value, dtype, 1)
                if value.numel() != M:
                    raise ValueError(f"{name} must have M entries")
                keep.append(value)
                return conv(0), value.data_ptr()
            return conv(value), None

        c.temperature, c.temperature_rows = split("temperature", self.temperature, torch.float32, float)
        c.top_k, c.top_k_rows = split("top_k", self.top_k, torch.int32, int)
        c.top_p, c.top_p_rows = split("top_p", self.top_p, torch.float32, float)
        c.min_p, c.min_p_rows = split("min_p", self.min_p, torch.float32, float)
        c.seed = self.seed & 0xFFFFFFFFFFFFFFFF
        if isinstance(self.offset, torch.Tensor):
            if self.offset.device.type != "cuda" or self.offset.numel() != 1 or \
                    self.offset.element_size() != 8 or not self.offset.is_contiguous():
                raise ValueError("offset tensor must be one contiguous 64-bit integer on the GPU")
            c.offset, c.offset_device = 0, self.offset.data_ptr()
            keep.append(self.offset)
        else:
            c.offset, c.offset_device = int(self.offset) & 0xFFFFFFFFFFFFFFFF, None
        c.tokens = tokens.data_ptr()
        c.kept = kept.data_ptr() if kept is not None else None
        c._keep = keep
        return c


def _opts(chunk_rows, score_events=None, lse=None, allowed=None, sampling=None):
    """score_events: None or (start, stop) hipEvent_t handles recorded at the
    scoring kernel's start and end.  lse: None or a float32 [M] GPU tensor
    that receives each row's log-sum-exp.  allowed: None or an int32
    [M, ceil(V/32)] GPU bitmask (bit 1 = allowed).  sampling: None or a
    _SamplingC."""
    lp = lse.data_ptr() if lse is not None else None
    ap = allowed.data_ptr() if allowed is not None else None
    sp = ctypes.pointer(sampling) if sampling is not None else None
    if score_events is None:
        o = _Options(int(chunk_rows), 0, None, lp, ap, sp)
    else:
        start, stop = (e.value if isinstance(e, ctypes.c_void_p) else int(e) for e in score_events)
        arr = (ctypes.c_void_p * 2)(start, stop)
        o = _Options(int(chunk_rows), 0, ctypes.cast(arr, ctypes.c_void_p), lp, ap, sp)
        o._events = arr  # keep the array alive as long as the options
    o._sampling = sampling
    return o


def _draw(sampling, dev, M, tokens, kept):
    """(C struct, tokens tensor) of a call's draw, or (None, None)."""
    if sampling is None:
        if tokens is not None or kept is not None:
            raise ValueError("tokens / kept need sampling=Sampling(...)")
        return None, None
    if not isinstance(sampling, Sampling):
        raise TypeError("sampling must be a Sampling")
    if tokens is None:
        tokens = torch.empty(M, dtype=torch.int64, device=dev)
    else:
        _need_cuda("tokens", tokens, torch.int64, 1)
        if tokens.numel() != M:
            raise ValueError("tokens must have M entries")
    if kept is not None:
        _need_cuda("kept", kept, torch.int32, 1)
        if kept.numel() != M:
            raise ValueError("kept must have M entries")
    return sampling._c(M, tokens, kept), tokens


def _allowed_in(allowed, M, V):
    if allowed is None:
        return None
    _need_cuda("allowed", allowed, torch.int32, 2)
    if tuple(allowed.shape) != (M, (V + 31) // 32):
        raise ValueError("allowed must be int32 [M, ceil(V / 32)]")
    return allowed


def _lse_out(lse, M):
    if lse is None:
        return None
    _need_cuda("lse", lse, torch.float32, 1)
    if lse.numel() != M:
        raise ValueError("lse must have M entries")
    return lse


@functools.lru_cache(maxsize=256)
def workspace_bytes(M, V, k, chunk_rows=0):
    n = ctypes.c_size_t()
    o = _opts(chunk_rows)
    _check(_lib.lmtopk_workspace_bytes(M, V, k, ctypes.byref(o), ctypes.byref(n)))
    return n.value


@functools.lru_cache(maxsize=256)
def binary_plan(M, V, H, k, chunk_rows=0):
    """(chunk_rows, n_chunks, waves per chunk workgroup) that lm_head_topk_binary
    uses for these sizes; they never change a result."""
    c, n, w = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    o = _opts(chunk_rows)
    _check(_lib.lmtopk_binary_plan(M, V, H, k, ctypes.byref(o), ctypes.byref(c), ctypes.byref(n),
                                   ctypes.byref(w)))
    return c.value, n.value, w.value


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need_cuda(name, t, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _outputs(dev, M, k, out):
    if out is None:
        return (torch.empty((M, k), dtype=torch.float32, device=dev),
                torch.empty((M, k), dtype=torch.int64, device=dev))
    values, indices = out
    _need_cuda("values", values, torch.float32, 2)
    _need_cuda("indices", indices, torch.int64, 2)
    if tuple(values.shape) != (M, k) or tuple(indices.shape) != (M, k):
        raise ValueError("out tensors must be [M, k]")
    return values, indices


_WORKSPACES = {}


def workspace_init(workspace):
    """Zero-fill a uint8 GPU workspace with the library's own kernel on the
    current stream (graph-capture safe, unlike a memset)."""
    _need_cuda("workspace", workspace, torch.uint8)
    _check(_lib.lmtopk_workspace_init(_ptr(workspace), workspace.numel(), _stream(workspace)))
    return workspace


def new_workspace(M, V, k, chunk_rows=0, device=None):
    """A workspace for these sizes on `device` (default: the current GPU),
    ready for its first call (zero-filled by workspace_init).  The library
    keeps its first 65,792 bytes (completion counter and key histograms) zero
    between calls; a workspace passed to the entry points must come from here (or be
    prepared by workspace_init), and calls that share one must be ordered on
    one stream."""
    if device is None:
        device = torch.device("cuda", torch.cuda.current_device())
    ws = torch.empty(workspace_bytes(M, V, k, chunk_rows), dtype=torch.uint8, device=device)
    return workspace_init(ws)


def _workspace(dev, M, V, k, chunk_rows, workspace):
    need = workspace_bytes(M, V, k, chunk_rows)
    if workspace is None:
        # one buffer per (device, stream), grown on demand: calls on one
        # stream are ordered, so they can share it
        key = (dev.index, torch.cuda.current_stream(dev).cuda_stream)
        ws = _WORKSPACES.get(key)
        if ws is None or ws.numel() < need:
            ws = workspace_init(torch.empty(need, dtype=torch.uint8, device=dev))
            _WORKSPACES[key] = ws
        return ws
    _need_cuda("workspace", workspace, torch.uint8)
    if workspace.numel() < need:
        raise ValueError(f"workspace needs {need} bytes, got {workspace.numel()}")
    return workspace


def pack_binary(weight, group_size=GROUP_SIZE):
    """Pack a dense head [V, H] (fp32 or bf16) into (wq, wscale), layout version 1.

    wq: uint8 [V64/64, G, 64, 16] sign bits; wscale: float32 [V64/64, G4/4, 64, 4].
    """
    _need_cuda("weight", weight, ndim=2)
    if weight.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("weight must be float32 or bfloat16")
    V, H = weight.shape
    wq_b, ws_b = packed_bytes(V, H, group_size)
    T = -(-V // 64)
    G = H // group_size
    Q = -(-G // 4)
    wq = torch.empty((T, G, 64, 16), dtype=torch.uint8, device=weight.device)
    ws = torch.empty((T, Q, 64, 4), dtype=torch.float32, device=weight.device)
    assert wq.numel() == wq_b and ws.numel() * 4 == ws_b
    dt = _BF16 if weight.dtype == torch.bfloat16 else _F32
    _check(_lib.lmtopk_pack_binary(_ptr(weight), dt, V, H, group_size, _ptr(wq), _ptr(ws),
                                   _stream(weight)))
    return wq, ws


def lm_head_topk_binary(act_q, act_scale, wq, wscale, bias=None, group_size=GROUP_SIZE, k=50, *,
                        vocab_size=None, chunk_rows=0, out=None, workspace=None,
                        score_events=None, lse=None, allowed=None, sampling=None, tokens=None,
                        kept=None):
    """Exact top-k of the binary-head logits of each activation row.

    act_q int8 [M, H]; act_scale float32 [M]; (wq, wscale) from pack_binary;
    bias float32 [V] or None.  vocab_size V is required when bias is None
    (the packed arrays are padded to whole 64-row tiles).  lse: optional
    float32 [M] GPU tensor that receives each row's log-sum-exp over all V
    logits (values - lse are the top-k log-probabilities).  allowed:
    optional int32 [M, ceil(V/32)] bitmask, bit 1 = allowed; a disallowed
    entry's logit counts as -inf.  sampling: a Sampling to also draw one
    token per row (returned as a third tensor, int64 [M]; `tokens` may give
    it, `kept` an int32 [M] tensor for the keep-set sizes).  A workspace
    passed in must come from new_workspace.
    """
    _need_cuda("act_q", act_q, torch.int8, 2)
    _need_cuda("act_scale", act_scale, torch.float32, 1)
    _need_cuda("wq", wq)
    _need_cuda("wscale", wscale, torch.float32)
    M, H = act_q.shape
    if act_scale.numel() != M:
        raise ValueError("act_scale must have M entries")
    if bias is not None:
        _need_cuda("bias", bias, torch.float32, 1)
        V = bias.numel() if vocab_size is None else int(vocab_size)
        if bias.numel() != V:
            raise ValueError("bias must have V entries")
    elif vocab_size is None:
        raise ValueError("vocab_size is required when bias is None")
    else:
        V = int(vocab_size)
    wq_b, ws_b = packed_bytes(V, H, group_size)
    if wq.numel() * wq.element_size() != wq_b or wscale.numel() * 4 != ws_b:
        raise ValueError("wq / wscale sizes do not match a packed V x H head")
    dev = act_q.device
    values, indices = _outputs(dev, M, k, out)
    ws = _workspace(dev, M, V, k, chunk_rows, workspace)
    sc, tok = _draw(sampling, dev, M, tokens, kept)
    o = _opts(chunk_rows, score_events, _lse_out(lse, M), _allowed_in(allowed, M, V), sc)
    _check(_lib.lmtopk_binary(_ptr(act_q), _ptr(act_scale), _ptr(wq), _ptr(wscale), _ptr(bias),
                              M, V, H, group_size, k, _ptr(values), _ptr(indices), _ptr(ws),
                              ws.numel(), ctypes.byref(o), _stream(act_q)))
    return (values, indices) if tok is None else (values, indices, tok)


def lm_head_topk_dense(hidden, weight, k=50, bias=None, *, chunk_rows=0, out=None,
                       workspace=None, score_events=None, lse=None, allowed=None, sampling=None,
                       tokens=None, kept=None):
    """Exact top-k of hidden @ weight.T (+ bias); hidden and weight both fp32 or both bf16.
    lse: optional float32 [M] GPU tensor for each row's log-sum-exp; allowed:
    optional int32 [M, ceil(V/32)] bitmask (bit 1 = allowed); sampling,
    tokens, kept: as for lm_head_topk_binary."""
    _need_cuda("hidden", hidden, ndim=2)
    _need_cuda("weight", weight, ndim=2)
    if hidden.dtype != weight.dtype or hidden.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("hidden and weight must share dtype float32 or bfloat16")
    M, H = hidden.shape
    V, H2 = weight.shape
    if H2 != H:
        raise ValueError("hidden and weight disagree on H")
    if bias is not None:
        _need_cuda("bias", bias, torch.float32, 1)
        if bias.numel() != V:
            raise ValueError("bias must have V entries")
    dev = hidden.device
    values, indices = _outputs(dev, M, k, out)
    ws = _workspace(dev, M, V, k, chunk_rows, workspace)
    sc, tok = _draw(sampling, dev, M, tokens, kept)
    o = _opts(chunk_rows, score_events, _lse_out(lse, M), _allowed_in(allowed, M, V), sc)
    dt = _BF16 if hidden.dtype == torch.bfloat16 else _F32
    _check(_lib.lmtopk_dense(_ptr(hidden), _ptr(weight), dt, _ptr(bias), M, V, H, k,
                             _ptr(values), _ptr(indices), _ptr(ws), ws.numel(), ctypes.byref(o),
                             _stream(hidden)))
    return (values, indices) if tok is None else (values, indices, tok)


def topk_logits(logits, k, *, chunk_rows=0, out=None, workspace=None, score_events=None,
                lse=None, allowed=None, sampling=None, tokens=None, kept=None):
    """The selection stage alone: exact top-k of each row of fp32 logits [M, V].
    lse: optional float32 [M] GPU tensor for each row's log-sum-exp; allowed:
    optional int32 [M, ceil(V/32)] bitmask (bit 1 = allowed); sampling,
    tokens, kept: as for lm_head_topk_binary."""
    if not isinstance(logits, torch.Tensor) or logits.device.type != "cuda":
        raise ValueError("logits must be a GPU tensor")
    if logits.dtype != torch.float32 or logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be float32 [M, V] with unit stride along V")
    M, V = logits.shape
    ld = logits.stride(0) if M > 1 else V
    dev = logits.device
    values, indices = _outputs(dev, M, k, out)
    ws = _workspace(dev, M, V, k, chunk_rows, workspace)
    sc, tok = _draw(sampling, dev, M, tokens, kept)
    o = _opts(chunk_rows, score_events, _lse_out(lse, M), _allowed_in(allowed, M, V), sc)
    _check(_lib.lmtopk_select(_ptr(logits), M, V, ld, k, _ptr(values), _ptr(indices), _ptr(ws),
                              ws.numel(), ctypes.byref(o), _stream(logits)))
    return (values, indices) if tok is None else (values, indices, tok)


def sample(logits, temperature=1.0, top_k=50, top_p=1.0, min_p=0.0, seed=0, offset=0, *, k=None,
           allowed=None, kept=None):
    """One token per row of fp32 logits [M, V] (logits-processor page, section
    "API": sample(logits, temperature, top_k, top_p, min_p, seed, offset)),
    drawn from the exact top-k survivors, k = top_k unless given (a per-row
    top_k tensor needs k).  Returns tokens int64 [M]."""
    if k is None:
        if isinstance(top_k, torch.Tensor) or int(top_k) <= 0:
            raise ValueError("k is needed when top_k is per row or off")
        k = int(top_k)
    _, _, tok = topk_logits(logits, k, allowed=allowed, kept=kept,
                            sampling=Sampling(temperature, top_k, top_p, min_p, seed, offset))
    return tok
