"""Thin ctypes binding of libhla.so (the C ABI declared in include/hla.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory and the current
stream.  There is no CPU fallback: if the library is missing or no GPU is
present, the calls raise.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhla.so")

HLA_F32 = 0
HLA_BF16 = 1

STATUS = {
    0: "HLA_OK", 1: "HLA_ERR_NULL_POINTER", 2: "HLA_ERR_BAD_SHAPE", 3: "HLA_ERR_BAD_DTYPE",
    4: "HLA_ERR_MISALIGNED", 5: "HLA_ERR_UNSUPPORTED", 6: "HLA_ERR_WORKSPACE_TOO_SMALL",
    7: "HLA_ERR_ALIASING", 8: "HLA_ERR_HIP", 9: "HLA_ERR_BAD_VALUE",
}

EXPORTS = (
    "hla_status_string", "hla_version", "hla_fwd_chunk_summaries", "hla_scan_workspace_bytes",
    "hla_scan", "hla_scan_into", "hla_scan_run_length", "hla_scan_runs_workspace_bytes",
    "hla_scan_runs",
    "hla_fwd_span_chunks",
    "hla_fwd_output_workspace_bytes", "hla_fwd_output", "hla_fwd_workspace_bytes",
    "hla_fwd_p_bytes", "hla_fwd_chunk_summaries_p", "hla_fwd_output_from_p",
    "hla_fwd_p_workspace_bytes",
    "hla_fwd", "hla_fwd_noalloc_max_workspace_bytes", "hla_fwd_noalloc",
    "hla_decode_step", "hla_unmasked_chunk_summaries", "hla_unmasked_scan",
    "hla_unmasked_output", "hla_unmasked_fwd_workspace_bytes", "hla_unmasked_fwd",
    "hla_unmasked_decode_step", "hla_ahla_chunk_summaries", "hla_ahla_scan", "hla_ahla_output",
    "hla_ahla_fwd_workspace_bytes", "hla_ahla_fwd", "hla_ahla_decode_step",
    "hla_bwd_workspace_bytes", "hla_bwd",
    "hla3_workspace_bytes", "hla3_chunk_summaries", "hla3_scan", "hla3_fwd", "hla3_decode_step",
)


class HlaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
        ("d", ctypes.c_int32), ("dv", ctypes.c_int32), ("chunk", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("normalize", ctypes.c_int32), ("eps", ctypes.c_float),
        ("gamma", ctypes.c_void_p),
    ]


class State(ctypes.Structure):
    _fields_ = [("S", ctypes.c_void_p), ("C", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("G", ctypes.c_void_p), ("h", ctypes.c_void_p)]


class AhlaState(ctypes.Structure):
    _fields_ = [("P", ctypes.c_void_p), ("m", ctypes.c_void_p), ("E", ctypes.c_void_p),
                ("n", ctypes.c_void_p), ("X", ctypes.c_void_p)]


class Summary3(ctypes.Structure):
    _fields_ = [(x, ctypes.c_void_p) for x in ("S", "Q", "P", "m", "V", "Z", "z", "R", "r")]


class State3(ctypes.Structure):
    _fields_ = [(x, ctypes.c_void_p) for x in ("S", "P", "m", "R", "r")]


_lib = None


def lib():
    """Load libhla.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                           "(run `python -m causal_prefix_scan_amd.build_lib`)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    pp, ps = ctypes.POINTER(Problem), ctypes.POINTER(State)
    L.hla_status_string.argtypes, L.hla_status_string.restype = [ctypes.c_int], ctypes.c_char_p
    L.hla_version.argtypes, L.hla_version.restype = [], ctypes.c_char_p
    L.hla_fwd_chunk_summaries.argtypes = [pp, vp, vp, vp, ps, vp]
    L.hla_scan_workspace_bytes.argtypes, L.hla_scan_workspace_bytes.restype = [pp], sz
    L.hla_scan.argtypes = [pp, ps, ps, vp, sz, vp]
    L.hla_scan_into.argtypes = [pp, ps, ps, ps, vp, sz, vp]
    L.hla_scan_run_length.argtypes, L.hla_scan_run_length.restype = [pp], i32
    L.hla_fwd_span_chunks.argtypes, L.hla_fwd_span_chunks.restype = [pp], i32
    L.hla_scan_runs_workspace_bytes.argtypes, L.hla_scan_runs_workspace_bytes.restype = [pp], sz
    L.hla_scan_runs.argtypes = [pp, ps, ps, vp, sz, vp]
    L.hla_fwd_output_workspace_bytes.argtypes, L.hla_fwd_output_workspace_bytes.restype = [pp], sz
    L.hla_fwd_output.argtypes = [pp, vp, vp, vp, ps, vp, vp, vp, sz, vp]
    L.hla_fwd_workspace_bytes.argtypes, L.hla_fwd_workspace_bytes.restype = [pp], sz
    L.hla_fwd_p_bytes.argtypes, L.hla_fwd_p_bytes.restype = [pp], sz
    L.hla_fwd_p_workspace_bytes.argtypes, L.hla_fwd_p_workspace_bytes.restype = [pp], sz
    L.hla_fwd_chunk_summaries_p.argtypes = [pp, vp, vp, vp, ps, vp, vp]
    L.hla_fwd_output_from_p.argtypes = [pp, vp, vp, vp, ps, vp, vp, vp]
    L.hla_fwd.argtypes = [pp, vp, vp, vp, vp, vp, ps, vp, sz, vp]
    L.hla_fwd_noalloc_max_workspace_bytes.argtypes = []
    L.hla_fwd_noalloc_max_workspace_bytes.restype = sz
    L.hla_fwd_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, ps, vp]
    L.hla_decode_step.argtypes = [i32, i32, i32, i32, i32, i32, f32, vp, vp, vp, vp, ps, vp, vp, vp]
    L.hla_unmasked_fwd_workspace_bytes.argtypes = [pp]
    L.hla_unmasked_fwd_workspace_bytes.restype = sz
    L.hla_unmasked_fwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.hla_unmasked_chunk_summaries.argtypes = [pp, vp, vp, vp, ps, vp]
    L.hla_unmasked_scan.argtypes = [pp, ps, vp]
    L.hla_unmasked_output.argtypes = [pp, vp, vp, vp, ps, vp, vp, vp]
    L.hla_unmasked_decode_step.argtypes = L.hla_decode_step.argtypes
    pa = ctypes.POINTER(AhlaState)
    L.hla_ahla_chunk_summaries.argtypes = [pp, vp, vp, vp, pa, vp]
    L.hla_ahla_scan.argtypes = [pp, pa, vp]
    L.hla_ahla_output.argtypes = [pp, vp, vp, vp, pa, vp, vp, vp]
    L.hla_ahla_fwd_workspace_bytes.argtypes, L.hla_ahla_fwd_workspace_bytes.restype = [pp], sz
    L.hla_ahla_fwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.hla_ahla_decode_step.argtypes = [i32, i32, i32, i32, i32, i32, f32, vp, vp, vp, vp, pa, vp, vp, vp]
    L.hla_bwd_workspace_bytes.argtypes, L.hla_bwd_workspace_bytes.restype = [pp], sz
    L.hla_bwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    p3s, p3t = ctypes.POINTER(Summary3), ctypes.POINTER(State3)
    L.hla3_workspace_bytes.argtypes, L.hla3_workspace_bytes.restype = [pp], sz
    L.hla3_chunk_summaries.argtypes = [pp, vp, vp, vp, p3s, vp, sz, vp]
    L.hla3_scan.argtypes = [pp, p3s, p3t, vp]
    L.hla3_fwd.argtypes = [pp, vp, vp, vp, vp, vp, p3t, vp, sz, vp]
    L.hla3_decode_step.argtypes = [i32, i32, i32, i32, i32, i32, f32, vp, vp, vp, vp, p3t, vp, vp, vp]
    for name in ("hla3_chunk_summaries", "hla3_scan", "hla3_fwd", "hla3_decode_step"):
        getattr(L, name).restype = ctypes.c_int
    for name in ("hla_fwd_chunk_summaries", "hla_scan", "hla_scan_runs", "hla_fwd_output",
                 "hla_fwd_chunk_summaries_p", "hla_fwd_output_from_p",
                 "hla_fwd", "hla_fwd_noalloc", "hla_decode_step", "hla_unmasked_fwd", "hla_unmasked_chunk_summaries",
                 "hla_unmasked_scan", "hla_unmasked_output", "hla_unmasked_decode_step",
                 "hla_ahla_chunk_summaries", "hla_ahla_scan", "hla_ahla_output", "hla_ahla_fwd",
                 "hla_ahla_decode_step", "hla_bwd"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def status_string(status):
    return lib().hla_status_string(int(status)).decode()


def version():
    return lib().hla_version().decode()


def _check(status, where):
    if status != 0:
        raise HlaError(status, where)


# ----------------------------------------------------------------------------
# torch-facing wrappers
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return HLA_BF16
    if t.dtype == torch.float32:
        return HLA_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _need_cuda(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise RuntimeError("HLA kernels need CUDA/HIP tensors (no CPU path)")
        if not t.is_contiguous():
            raise RuntimeError("HLA kernels need contiguous tensors")


def make_problem(q, v, chunk, gamma=None, normalize=False, eps=0.0):
    B, H, T, d = q.shape
    return Problem(B, H, T, d, v.shape[3], int(chunk), _dtype_code(q), int(bool(normalize)),
                   float(eps), None if gamma is None else gamma.data_ptr())


def _state_struct(st):
    if st is None:
        return None
    return State(*(None if st.get(k) is None else st[k].data_ptr() for k in ("S", "C", "m", "G", "h")))


def alloc_state(lead, d, dv, device):
    """fp32 state / summary tensors with leading dims `lead` (a tuple)."""
    torch = _torch()
    z = lambda *s: torch.zeros(*lead, *s, dtype=torch.float32, device=device)
    return {"S": z(d, d), "C": z(d, dv), "m": z(d), "G": z(d, dv), "h": z(d)}


def fwd_chunk_summaries(q, k, v, chunk, gamma=None, out=None):
    """Segment summaries [B, H, n, ...] (fp32 dict S, C, m, G, h)."""
    _need_cuda(q, k, v, gamma)
    B, H, T, d = q.shape
    p = make_problem(q, v, chunk, gamma)
    if out is None:
        out = alloc_state((B, H, T // chunk), d, v.shape[3], q.device)
    st = _state_struct(out)
    _check(lib().hla_fwd_chunk_summaries(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                         ctypes.byref(st), _stream()), "hla_fwd_chunk_summaries")
    return out


def scan(summaries, q_shape, dv, chunk, dtype_code, gamma=None, want_total=False):
    """In-place exclusive scan of `summaries`; returns the inclusive total (or None)."""
    torch = _torch()
    B, H, T, d = q_shape
    p = Problem(B, H, T, d, dv, int(chunk), dtype_code, 0, 0.0,
                None if gamma is None else gamma.data_ptr())
    dev = summaries["S"].device
    total = alloc_state((B, H), d, dv, dev) if want_total else None
    nbytes = lib().hla_scan_workspace_bytes(ctypes.byref(p))
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    st = _state_struct(summaries)
    tt = _state_struct(total)
    _check(lib().hla_scan(ctypes.byref(p), ctypes.byref(st),
                          ctypes.byref(tt) if tt is not None else None,
                          _ptr(ws), ctypes.c_size_t(nbytes), _stream()), "hla_scan")
    return total


def scan_into(summaries, q_shape, dv, chunk, dtype_code, gamma=None, want_total=False,
              prefixes=None):
    """hla_scan_into: the exclusive prefixes of `summaries` (only read) in a
    new state dict (or `prefixes`); returns (prefixes, inclusive total or None)."""
    torch = _torch()
    B, H, T, d = q_shape
    p = Problem(B, H, T, d, dv, int(chunk), dtype_code, 0, 0.0,
                None if gamma is None else gamma.data_ptr())
    dev = summaries["S"].device
    if prefixes is None:
        prefixes = alloc_state((B, H, T // int(chunk)), d, dv, dev)
    total = alloc_state((B, H), d, dv, dev) if want_total else None
    nbytes = lib().hla_scan_workspace_bytes(ctypes.byref(p))
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    st, po, tt = _state_struct(summaries), _state_struct(prefixes), _state_struct(total)
    _check(lib().hla_scan_into(ctypes.byref(p), ctypes.byref(st), ctypes.byref(po),
                               ctypes.byref(tt) if tt is not None else None,
                               _ptr(ws), ctypes.c_size_t(nbytes), _stream()), "hla_scan_into")
    return prefixes, total


def scan_run_length(T, chunk):
    """Segments per run of the blocked scan for n = T // chunk segments (host only)."""
    p = Problem(1, 1, int(T), 16, 16, int(chunk), HLA_F32, 0, 0.0, None)
    return int(lib().hla_scan_run_length(ctypes.byref(p)))


def fwd_span_chunks(q, v, chunk, gamma=None):
    """Chunks per span that hla_fwd's kernels walk (see hla_fwd_span_chunks)."""
    p = make_problem(q, v, chunk, gamma)
    return int(lib().hla_fwd_span_chunks(ctypes.byref(p)))


def scan_runs(summaries, q_shape, dv, chunk, dtype_code, gamma=None):
    """Exclusive prefixes at the run starts [B, H, runs, ...]; `summaries` is only read."""
    torch = _torch()
    B, H, T, d = q_shape
    p = Problem(B, H, T, d, dv, int(chunk), dtype_code, 0, 0.0,
                None if gamma is None else gamma.data_ptr())
    dev = summaries["S"].device
    n = T // chunk
    R = int(lib().hla_scan_run_length(ctypes.byref(p)))
    runs = (n + R - 1) // R
    out = alloc_state((B, H, runs), d, dv, dev)
    nbytes = lib().hla_scan_runs_workspace_bytes(ctypes.byref(p))
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    st, rt = _state_struct(summaries), _state_struct(out)
    _check(lib().hla_scan_runs(ctypes.byref(p), ctypes.byref(st), ctypes.byref(rt), _ptr(ws),
                               ctypes.c_size_t(nbytes), _stream()), "hla_scan_runs")
    return out


def fwd_output(q, k, v, prefixes, chunk, gamma=None, normalize=False, eps=0.0, want_den=False):
    """Outputs from exclusive prefixes: (o [B,H,T,dv] fp32, den [B,H,T] or None)."""
    torch = _torch()
    _need_cuda(q, k, v, gamma)
    B, H, T, d = q.shape
    p = make_problem(q, v, chunk, gamma, normalize, eps)
    o = torch.empty(B, H, T, v.shape[3], dtype=torch.float32, device=q.device)
    den = torch.empty(B, H, T, dtype=torch.float32, device=q.device) if want_den else None
    st = _state_struct(prefixes)
    _check(lib().hla_fwd_output(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(st),
                                _ptr(o), _ptr(den), None, ctypes.c_size_t(0), _stream()),
           "hla_fwd_output")
    return o, den


def fwd_workspace(q, v, chunk, gamma=None, with_p=True):
    """hla_fwd's workspace: with room for the segment-local p where the shape
    has that path (with_p), else the minimum (summaries and scan scratch)."""
    torch = _torch()
    p = make_problem(q, v, chunk, gamma)
    f = lib().hla_fwd_p_workspace_bytes if with_p else lib().hla_fwd_workspace_bytes
    nbytes = f(ctypes.byref(p))
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)


def p_bytes(q, v, chunk):
    """Bytes of the segment-local p (hla_fwd_p_bytes; 0 without that path)."""
    return lib().hla_fwd_p_bytes(ctypes.byref(make_problem(q, v, chunk)))


def fwd_chunk_summaries_p(q, k, v, chunk, gamma=None, out=None, plocal=None):
    """Segment summaries and the segment-local p: (summaries dict, plocal bf16 tensor)."""
    torch = _torch()
    _need_cuda(q, k, v, gamma)
    B, H, T, d = q.shape
    p = make_problem(q, v, chunk, gamma)
    if out is None:
        out = alloc_state((B, H, T // chunk), d, v.shape[3], q.device)
    if plocal is None:
        plocal = torch.empty(max(p_bytes(q, v, chunk), 16) // 2, dtype=torch.bfloat16, device=q.device)
    st = _state_struct(out)
    _check(lib().hla_fwd_chunk_summaries_p(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                           ctypes.byref(st), _ptr(plocal), _stream()),
           "hla_fwd_chunk_summaries_p")
    return out, plocal


def fwd_output_from_p(q, v, plocal, prefixes, chunk, gamma=None, normalize=False, eps=0.0,
                      want_den=False):
    """Outputs from the exclusive prefixes and the segment-local p: (o, den or None)."""
    torch = _torch()
    _need_cuda(q, v, plocal, gamma)
    B, H, T, d = q.shape
    p = make_problem(q, v, chunk, gamma, normalize, eps)
    o = torch.empty(B, H, T, v.shape[3], dtype=torch.float32, device=q.device)
    den = torch.empty(B, H, T, dtype=torch.float32, device=q.device) if want_den else None
    st = _state_struct(prefixes)
    _check(lib().hla_fwd_output_from_p(ctypes.byref(p), _ptr(q), _ptr(v), _ptr(plocal),
                                       ctypes.byref(st), _ptr(o), _ptr(den), _stream()),
           "hla_fwd_output_from_p")
    return o, den


def fwd(q, k, v, chunk, gamma=None, normalize=False, eps=0.0, want_den=False, want_state=False,
        workspace=None, o=None, den=None):
    """Whole chunk-parallel forward: (o, den or None, final state dict or None)."""
    torch = _torch()
    _need_cuda(q, k, v, gamma)
    B, H, T, d = q.shape
    dv = v.shape[3]
    p = make_problem(q, v, chunk, gamma, normalize, eps)
    if o is None:
        o = torch.empty(B, H, T, dv, dtype=torch.float32, device=q.device)
    if den is None and want_den:
        den = torch.empty(B, H, T, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = fwd_workspace(q, v, chunk, gamma)
    final = alloc_state((B, H), d, dv, q.device) if want_state else None
    fs = _state_struct(final)
    _check(lib().hla_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(den),
                         ctypes.byref(fs) if fs is not None else None, _ptr(workspace),
                         ctypes.c_size_t(workspace.numel()), _stream()), "hla_fwd")
    return o, den, final


def fwd_noalloc(q, k, v, chunk, gamma=None, normalize=False, eps=0.0, want_den=False,
                want_state=False, o=None, den=None):
    """hla_fwd_noalloc: the forward with the library's own fixed scratch (no
    workspace argument).  Returns (o, den or None, final state dict or None)."""
    torch = _torch()
    _need_cuda(q, k, v, gamma)
    B, H, T, d = q.shape
    dv = v.shape[3]
    p = make_problem(q, v, chunk, gamma, normalize, eps)
    if o is None:
        o = torch.empty(B, H, T, dv, dtype=torch.float32, device=q.device)
    if den is None and want_den:
        den = torch.empty(B, H, T, dtype=torch.float32, device=q.device)
    final = alloc_state((B, H), d, dv, q.device) if want_state else None
    fs = _state_struct(final)
    _check(lib().hla_fwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(den),
                                 ctypes.byref(fs) if fs is not None else None, _stream()),
           "hla_fwd_noalloc")
    return o, den, final


def alloc_moments(lead, d, dv, device):
    """fp32 S, C, m tensors with leading dims `lead` (the unmasked variant's state)."""
    torch = _torch()
    z = lambda *s: torch.zeros(*lead, *s, dtype=torch.float32, device=device)
    return {"S": z(d, d), "C": z(d, dv), "m": z(d)}


def unmasked_chunk_summaries(q, k, v, chunk, gamma=None, out=None):
    """Segment moments of the unmasked variant [B, H, n, ...] (fp32 dict S, C, m)."""
    _need_cuda(q, k, v, gamma)
    B, H, T, d = q.shape
    p = make_problem(q, v, chunk, gamma)
    if out is None:
        out = alloc_moments((B, H, T // chunk), d, v.shape[3], q.device)
    st = _state_struct(out)
    _check(lib().hla_unmasked_chunk_summaries(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                              ctypes.byref(st), _stream()),
           "hla_unmasked_chunk_summaries")
    return out


def unmasked_scan(moments, q_shape, dv, chunk, dtype_code, gamma=None):
    """In-place exclusive scan of the unmasked variant's segment moments."""
    B, H, T, d = q_shape
    p = Problem(B, H, T, d, dv, int(chunk), dtype_code, 0, 0.0,
                None if gamma is None else gamma.data_ptr())
    st = _state_struct(moments)
    _check(lib().hla_unmasked_scan(ctypes.byref(p), ctypes.byref(st), _stream()), "hla_unmasked_scan")


def unmasked_output(q, k, v, prefixes, chunk, gamma=None, normalize=False, eps=0.0, want_den=False):
    """Outputs of the unmasked variant from the exclusive prefixes: (o, den or None)."""
    torch = _torch()
    _need_cuda(q, k, v, gamma)
    B, H, T, d = q.shape
    dv = v.shape[3]
    p = make_problem(q, v, chunk, gamma, normalize, eps)
    o = torch.empty(B, H, T, dv, dtype=torch.float32, device=q.device)
    den = torch.empty(B, H, T, dtype=torch.float32, device=q.device) if want_den else None
    st = _state_struct(prefixes)
    _check(lib().hla_unmasked_output(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(st),
                                     _ptr(o), _ptr(den), _stream()), "hla_unmasked_output")
    return o, den


def unmasked_fwd(q, k, v, chunk, gamma=None, normalize=False, eps=0.0, want_den=False,
                 workspace=None, o=None, den=None):
    """The unmasked variant o = q^T S C (segment moments, scan, outputs on one
    stream): (o [B, H, T, dv] fp32, den [B, H, T] or None)."""
    torch = _torch()
    _need_cuda(q, k, v, gamma)
    B, H, T, d = q.shape
    dv = v.shape[3]
    p = make_problem(q, v, chunk, gamma, normalize, eps)
    if o is None:
        o = torch.empty(B, H, T, dv, dtype=torch.float32, device=q.device)
    if den is None and want_den:
        den = torch.empty(B, H, T, dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = lib().hla_unmasked_fwd_workspace_bytes(ctypes.byref(p))
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _check(lib().hla_unmasked_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(den),
                                  _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream()),
           "hla_unmasked_fwd")
    return o, den


def bwd(q, k, v, dout, chunk, gamma=None, workspace=None, dq=None, dk=None, dv=None,
        normalize=False, eps=0.0):
    """Gradients of the masked forward (unnormalised, or num / (den + eps) with
    normalize) for the upstream gradient dout [B, H, T, dv] (fp32):
    (dq, dk [B, H, T, d], dv [B, H, T, dv]) fp32."""
    torch = _torch()
    _need_cuda(q, k, v, dout, gamma)
    if dout.dtype != torch.float32:
        raise RuntimeError("dout must be float32")
    B, H, T, d = q.shape
    e = v.shape[3]
    p = make_problem(q, v, chunk, gamma, normalize, eps)
    if dq is None:
        dq = torch.empty(B, H, T, d, dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.empty(B, H, T, d, dtype=torch.float32, device=q.device)
    if dv is None:
        dv = torch.empty(B, H, T, e, dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = lib().hla_bwd_workspace_bytes(ctypes.byref(p))
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _check(lib().hla_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk),
                         _ptr(dv), _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream()),
           "hla_bwd")
    return dq, dk, dv


def decode_step(q, k, v, state, gamma=None, normalize=False, eps=0.0, o=None, den=None):
    """One decode step; q, k [N, H, d], v [N, H, dv]; `state` is updated in place.
    Returns (o [N, H, dv] fp32, den [N, H] or None)."""
    torch = _torch()
    _need_cuda(q, k, v, gamma)
    N, H, d = q.shape
    dv = v.shape[2]
    if o is None:
        o = torch.empty(N, H, dv, dtype=torch.float32, device=q.device)
    st = _state_struct(state)
    _check(lib().hla_decode_step(N, H, d, dv, _dtype_code(q), int(bool(normalize)), float(eps),
                                 _ptr(gamma), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(st),
                                 _ptr(o), _ptr(den), _stream()), "hla_decode_step")
    return o, den


def unmasked_decode_step(q, k, v, state, gamma=None, normalize=False, eps=0.0, o=None, den=None):
    """One decode step of the unmasked variant; q, k [N, H, d], v [N, H, dv];
    `state` (dict with S, C, m) is updated in place.  Returns (o, den or None)."""
    torch = _torch()
    _need_cuda(q, k, v, gamma)
    N, H, d = q.shape
    dv = v.shape[2]
    if o is None:
        o = torch.empty(N, H, dv, dtype=torch.float32, device=q.device)
    st = _state_struct(state)
    _check(lib().hla_unmasked_decode_step(N, H, d, dv, _dtype_code(q), int(bool(normalize)),
                                          float(eps), _ptr(gamma), _ptr(q), _ptr(k), _ptr(v),
                                          ctypes.byref(st), _ptr(o), _ptr(den), _stream()),
           "hla_unmasked_decode_step")
    return o, den


def alloc_ahla_state(lead, d, dv, device):
    """fp32 AHLA summary tensors P, m, E, n, X with leading dims `lead`."""
    torch = _torch()
    z = lambda *s: torch.zeros(*lead, *s, dtype=torch.float32, device=device)
    return {"P": z(d, dv), "m": z(d), "E": z(d, dv), "n": z(d), "X": z(d, d)}


def _ahla_struct(st):
    return AhlaState(*(None if st.get(k) is None else st[k].data_ptr()
                       for k in ("P", "m", "E", "n", "X")))


def ahla_chunk_summaries(q, k, v, chunk, gamma=None, out=None):
    """AHLA segment summaries [B, H, n, ...] (fp32 dict P, m, E, n, X)."""
    _need_cuda(q, k, v, gamma)
    B, H, T, d = q.shape
    p = make_problem(q, v, chunk, gamma)
    if out is None:
        out = alloc_ahla_state((B, H, T // chunk), d, v.shape[3], q.device)
    st = _ahla_struct(out)
    _check(lib().hla_ahla_chunk_summaries(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                          ctypes.byref(st), _stream()), "hla_ahla_chunk_summaries")
    return out


def ahla_scan(summaries, q_shape, dv, chunk, dtype_code, gamma=None):
    """In-place exclusive scan of AHLA summaries."""
    B, H, T, d = q_shape
    p = Problem(B, H, T, d, dv, int(chunk), dtype_code, 0, 0.0,
                None if gamma is None else gamma.data_ptr())
    st = _ahla_struct(summaries)
    _check(lib().hla_ahla_scan(ctypes.byref(p), ctypes.byref(st), _stream()), "hla_ahla_scan")


def ahla_output(q, k, v, prefixes, chunk, gamma=None, normalize=False, eps=0.0, want_den=False):
    """AHLA outputs from the exclusive prefixes: (o, den or None)."""
    torch = _torch()
    _need_cuda(q, k, v, gamma)
    B, H, T, d = q.shape
    dv = v.shape[3]
    p = make_problem(q, v, chunk, gamma, normalize, eps)
    o = torch.empty(B, H, T, dv, dtype=torch.float32, device=q.device)
    den = torch.empty(B, H, T, dtype=torch.float32, device=q.device) if want_den else None
    st = _ahla_struct(prefixes)
    _check(lib().hla_ahla_output(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(st),
                                 _ptr(o), _ptr(den), _stream()), "hla_ahla_output")
    return o, den


def ahla_fwd(q, k, v, chunk, gamma=None, normalize=False, eps=0.0, want_den=False,
             workspace=None, o=None, den=None):
    """The AHLA forward (summaries, scan, outputs on one stream): (o, den or None)."""
    torch = _torch()
    _need_cuda(q, k, v, gamma)
    B, H, T, d = q.shape
    dv = v.shape[3]
    p = make_problem(q, v, chunk, gamma, normalize, eps)
    if o is None:
        o = torch.empty(B, H, T, dv, dtype=torch.float32, device=q.device)
    if den is None and want_den:
        den = torch.empty(B, H, T, dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = lib().hla_ahla_fwd_workspace_bytes(ctypes.byref(p))
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _check(lib().hla_ahla_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(den),
                              _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream()),
           "hla_ahla_fwd")
    return o, den


def ahla_decode_step(q, k, v, state, gamma=None, normalize=False, eps=0.0, o=None, den=None):
    """One AHLA decode step; q, k [N, H, d], v [N, H, dv]; `state` (dict with
    P, m, E, n) is updated in place.  Returns (o [N, H, dv] fp32, den or None)."""
    torch = _torch()
    _need_cuda(q, k, v, gamma)
    N, H, d = q.shape
    dv = v.shape[2]
    if o is None:
        o = torch.empty(N, H, dv, dtype=torch.float32, device=q.device)
    st = _ahla_struct(state)
    _check(lib().hla_ahla_decode_step(N, H, d, dv, _dtype_code(q), int(bool(normalize)), float(eps),
                                      _ptr(gamma), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(st),
                                      _ptr(o), _ptr(den), _stream()), "hla_ahla_decode_step")
    return o, den


# ---- third order ------------------------------------------------------------

SUMMARY3_FIELDS = ("S", "Q", "P", "m", "V", "Z", "z", "R", "r")
STATE3_FIELDS = ("S", "P", "m", "R", "r")


def alloc_summary3(lead, d, dv, device):
    """fp32 third-order segment summaries with leading dims `lead`."""
    torch = _torch()
    shapes = {"S": (d, d), "Q": (d, d), "V": (d, d), "P": (d, dv), "Z": (d, dv), "R": (d, dv),
              "m": (d,), "z": (d,), "r": (d,)}
    return {x: torch.zeros(*lead, *shapes[x], dtype=torch.float32, device=device)
            for x in SUMMARY3_FIELDS}


def alloc_state3(lead, d, dv, device):
    """fp32 third-order decode state (S, P, m, R, r) with leading dims `lead`."""
    torch = _torch()
    shapes = {"S": (d, d), "P": (d, dv), "m": (d,), "R": (d, dv), "r": (d,)}
    return {x: torch.zeros(*lead, *shapes[x], dtype=torch.float32, device=device)
            for x in STATE3_FIELDS}


def _s3(st):
    return None if st is None else Summary3(*(_ptr(st[x]) for x in SUMMARY3_FIELDS))


def _t3(st):
    return None if st is None else State3(*(_ptr(st.get(x)) for x in STATE3_FIELDS))


def _ws3(p, device):
    torch = _torch()
    n = lib().hla3_workspace_bytes(ctypes.byref(p))
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def hla3_chunk_summaries(q, k, v, chunk, gamma=None):
    """Third-order segment summaries [B, H, n, ...] (dict of fp32 tensors)."""
    _need_cuda(q, k, v, gamma)
    B, H, T, d = q.shape
    p = make_problem(q, v, chunk, gamma)
    out = alloc_summary3((B, H, T // chunk), d, v.shape[3], q.device)
    ws = _ws3(p, q.device)
    _check(lib().hla3_chunk_summaries(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(_s3(out)),
                                      _ptr(ws), ctypes.c_size_t(ws.numel()), _stream()),
           "hla3_chunk_summaries")
    return out


def hla3_scan(summaries, q, v, chunk, gamma=None, want_total=False):
    """In place: S, P, m, R, r become exclusive prefixes; returns the inclusive
    totals (dict) or None."""
    _need_cuda(q, v, gamma)
    B, H, T, d = q.shape
    p = make_problem(q, v, chunk, gamma)
    total = alloc_state3((B, H), d, v.shape[3], q.device) if want_total else None
    t = _t3(total)
    _check(lib().hla3_scan(ctypes.byref(p), ctypes.byref(_s3(summaries)),
                           ctypes.byref(t) if t is not None else None, _stream()), "hla3_scan")
    return total


def hla3_fwd(q, k, v, chunk, gamma=None, normalize=False, eps=0.0, want_den=False, want_state=False,
             o=None, den=None):
    """Third-order chunk-parallel forward: (o, den or None, final state or None)."""
    torch = _torch()
    _need_cuda(q, k, v, gamma)
    B, H, T, d = q.shape
    dv = v.shape[3]
    p = make_problem(q, v, chunk, gamma, normalize, eps)
    if o is None:
        o = torch.empty(B, H, T, dv, dtype=torch.float32, device=q.device)
    if den is None and want_den:
        den = torch.empty(B, H, T, dtype=torch.float32, device=q.device)
    final = alloc_state3((B, H), d, dv, q.device) if want_state else None
    t = _t3(final)
    ws = _ws3(p, q.device)
    _check(lib().hla3_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(den),
                          ctypes.byref(t) if t is not None else None, _ptr(ws),
                          ctypes.c_size_t(ws.numel()), _stream()), "hla3_fwd")
    return o, den, final


def hla3_decode_step(q, k, v, state, gamma=None, normalize=False, eps=0.0, o=None, den=None):
    """One third-order decode step; q, k [N, H, d], v [N, H, dv]; `state`
    (S, P, m, R, r) is updated in place.  Returns (o, den or None)."""
    torch = _torch()
    _need_cuda(q, k, v, gamma)
    N, H, d = q.shape
    dv = v.shape[2]
    if o is None:
        o = torch.empty(N, H, dv, dtype=torch.float32, device=q.device)
    t = _t3(state)
    _check(lib().hla3_decode_step(N, H, d, dv, _dtype_code(q), int(bool(normalize)), float(eps),
                                  _ptr(gamma), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(t), _ptr(o),
                                  _ptr(den), _stream()), "hla3_decode_step")
    return o, den
