"""MI355X (gfx950) scaled-dot-product-attention backward.

A thin ctypes binding of the C ABI declared in include/sdpa_bwd.h: argument marshalling only,
every step of the backward runs in the HIP kernels of libsdpa_bwd.so.  PyTorch supplies device
memory and streams.  The library is loaded on first use and the call fails loudly when it has not
been built (``python -m attention_backward_sdpa_amd.build``).
"""
import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsdpa_bwd.so")

OK, INVALID_ARG, UNSUPPORTED, WORKSPACE_TOO_SMALL, LAUNCH_FAILED, SCRATCH_TOO_SMALL = 0, 1, 2, 3, 4, 5
# the static device scratch of sdpa_bwd_noalloc (SDPA_BWD_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 256 << 20
BF16, FP16, FP32 = 0, 1, 2
# values of the `deterministic` argument (dQ routes); False / True are 0 / 1
DQ_ATOMIC, DQ_DETERMINISTIC, DQ_DS_PANELS, DQ_PARTIALS, DQ_RELAY = 0, 1, 2, 3, 4


class Layout(ctypes.Structure):
    """sdpa_bwd_layout: element strides (batch, head, seq) of a (B, H, S, D) tensor."""
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("seq", ctypes.c_int64)]



class Args(ctypes.Structure):
    """sdpa_bwd_args: every argument of one sdpa_bwd_run call."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("q", "k", "v", "o", "dO", "lse", "dq", "dk", "dv")] + \
        [(n, ctypes.c_int) for n in ("B", "Hq", "Hkv", "Sq", "Skv", "Dqk", "Dv")] + \
        [("scale", ctypes.c_float)] + \
        [(n, ctypes.c_int) for n in ("causal", "causal_bottom_right", "window_left",
                                     "window_right", "deterministic")] + \
        [("seq_q_lens", ctypes.c_void_p), ("seq_kv_lens", ctypes.c_void_p),
         ("layouts", ctypes.c_void_p), ("dtype", ctypes.c_int), ("sink", ctypes.c_void_p),
         ("dsink", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("bias_dtype", ctypes.c_int),
         ("bias_batch", ctypes.c_int), ("dbias", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
         ("workspace_bytes", ctypes.c_size_t), ("stream", ctypes.c_void_p),
         ("events", ctypes.c_void_p), ("dbias_io", ctypes.c_int)]


_lib = None


class SdpaBwdError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m attention_backward_sdpa_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.sdpa_bwd_workspace_size.argtypes = [i] * 11
    lib.sdpa_bwd_workspace_size.restype = sz
    lib.sdpa_bwd.argtypes = [vp] * 9 + [i] * 7 + [f, i, i, i, vp, vp]
    lib.sdpa_bwd.restype = i
    ex = [vp] * 9 + [i] * 7 + [f, i, i, i, vp, vp, i, i, vp, sz, vp]
    lib.sdpa_bwd_ex.argtypes = ex
    lib.sdpa_bwd_ex.restype = i
    lib.sdpa_bwd_noalloc.argtypes = [vp] * 9 + [i] * 7 + [f, i, i, i, vp, vp, i, i, vp]
    lib.sdpa_bwd_noalloc.restype = i
    lib.sdpa_bwd_ex_events.argtypes = ex + [vp]
    lib.sdpa_bwd_ex_events.restype = i
    lib.sdpa_bwd_flex.argtypes = ([vp] * 9 + [i] * 7 + [f, i, i, i, vp, vp, i, i, vp, i, vp, sz, vp,
                                                    vp])
    lib.sdpa_bwd_flex.restype = i
    lib.sdpa_bwd_preprocess.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.sdpa_bwd_preprocess.restype = i
    lib.sdpa_bwd_run.argtypes = [ctypes.POINTER(Args)]
    lib.sdpa_bwd_run.restype = i
    lib.sdpa_bwd_run_workspace_size.argtypes = [ctypes.POINTER(Args)]
    lib.sdpa_bwd_run_workspace_size.restype = sz
    lib.sdpa_bwd_nvfp4_qat.argtypes = [vp] * 9 + [i] * 5 + [f, i, i, vp, sz, vp, vp]
    lib.sdpa_bwd_nvfp4_qat.restype = i
    lib.sdpa_bwd_nvfp4_qat_workspace_size.argtypes = [i] * 7
    lib.sdpa_bwd_nvfp4_qat_workspace_size.restype = sz
    lib.sdpa_bwd_dq_route.argtypes = [i] * 8
    lib.sdpa_bwd_dq_route.restype = i
    lib.sdpa_bwd_run_dq_route.argtypes = [ctypes.POINTER(Args)]
    lib.sdpa_bwd_run_dq_route.restype = i
    lib.sdpa_bwd_status_string.argtypes = [i]
    lib.sdpa_bwd_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def library():
    """The loaded ctypes library (raises when it has not been built)."""
    return _load()


def status_string(status: int) -> str:
    return _load().sdpa_bwd_status_string(int(status)).decode()


def _check(status):
    if status != OK:
        raise SdpaBwdError(status, f"sdpa_bwd failed: {status_string(status)} (status {status})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _events(events):
    """Five torch.cuda.Event (or None entries) as the hipEvent_t array of the C ABI, or NULL."""
    if events is None:
        return None
    return (ctypes.c_void_p * 5)(*[ctypes.c_void_p(None if e is None else e.cuda_event)
                                   for e in events])


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def workspace_size(B, Hq, Hkv, Sq, Skv, Dqk, Dv, causal=False, window_left=-1,
                   deterministic=False, has_seqlens=False) -> int:
    """sdpa_bwd_workspace_size(): bytes of workspace a call with these arguments needs."""
    return int(_load().sdpa_bwd_workspace_size(B, Hq, Hkv, Sq, Skv, Dqk, Dv, int(causal),
                                               int(window_left), int(deterministic),
                                               int(has_seqlens)))


def dq_route(B, Hq, Hkv, Sq, Skv, Dqk, Dv, deterministic) -> int:
    """sdpa_bwd_dq_route(): the dQ route (DQ_ATOMIC, DQ_DS_PANELS, DQ_PARTIALS or DQ_RELAY) a call
    with these sizes takes, -1 for unsupported arguments."""
    return int(_load().sdpa_bwd_dq_route(int(B), int(Hq), int(Hkv), int(Sq), int(Skv), int(Dqk),
                                         int(Dv), int(deterministic)))


def _dims(q, k, v):
    B, Hq, Sq, Dqk = q.shape
    _, Hkv, Skv, _ = k.shape
    Dv = v.shape[-1]
    return B, Hq, Hkv, Sq, Skv, Dqk, Dv


def sdpa_bwd(q, k, v, o, do, lse, dq, dk, dv, scale=None, causal=False, window_left=-1,
             deterministic=False, workspace=None, stream=None):
    """sdpa_bwd(): the plain entry point on torch tensors (bf16 BHSD, lse fp32 (B,Hq,Sq)).

    Outputs dq, dk, dv are written in place.  `workspace` is a uint8 device tensor of at least
    workspace_size(...) bytes.  Raises SdpaBwdError on a non-zero status.
    """
    dims = _dims(q, k, v)
    _check(_load().sdpa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                            _ptr(dk), _ptr(dv), *dims, -1.0 if scale is None else float(scale),
                            int(causal), int(window_left), int(deterministic), _ptr(workspace),
                            _stream_handle(stream)))


def _layouts(tensors):
    """Eight sdpa_bwd_layout entries from the tensors' strides (head dim must be contiguous)."""
    arr = (Layout * 8)()
    for x, t in enumerate(tensors):
        if t.dim() != 4 or t.stride(3) != 1:
            raise ValueError("sdpa_bwd_flex needs 4-D (B, H, S, D) tensors with a contiguous head dim")
        arr[x] = Layout(t.stride(0), t.stride(1), t.stride(2))
    return arr


def _io_dtype(q):
    import torch
    return FP16 if q.dtype == torch.float16 else BF16


def sdpa_bwd_ex(q, k, v, o, do, lse, dq, dk, dv, scale=None, causal=False, window_left=-1,
                deterministic=False, seq_q_lens=None, seq_kv_lens=None,
                causal_bottom_right=False, window_right=0, workspace=None, stream=None,
                events=None):
    """sdpa_bwd_ex() (or sdpa_bwd_ex_events() when `events` lists five torch.cuda.Event or
    None, a None entry not being recorded).  Tensors that are not all contiguous bf16 go through
    sdpa_bwd_flex with their own strides (any dense layout with a contiguous head dim)."""
    dims = _dims(q, k, v)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    head = [_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
            *dims, -1.0 if scale is None else float(scale), int(causal), int(window_left),
            int(deterministic), _ptr(seq_q_lens), _ptr(seq_kv_lens), int(causal_bottom_right),
            int(window_right)]
    tail = [_ptr(workspace), ws_bytes, _stream_handle(stream)]
    handles = None
    if events is not None:
        handles = (ctypes.c_void_p * 5)(
            *[ctypes.c_void_p(None if e is None else e.cuda_event) for e in events])
    lib = _load()
    tensors = (q, k, v, o, do, dq, dk, dv)
    if all(t.is_contiguous() for t in tensors) and _io_dtype(q) == BF16:
        if handles is None:
            _check(lib.sdpa_bwd_ex(*head, *tail))
        else:
            _check(lib.sdpa_bwd_ex_events(*head, *tail, handles))
    else:
        _check(lib.sdpa_bwd_flex(*head, _layouts(tensors), _io_dtype(q), *tail, handles))


def sdpa_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, scale=None, causal=False, window_left=-1,
                     deterministic=False, seq_q_lens=None, seq_kv_lens=None,
                     causal_bottom_right=False, window_right=0, stream=None):
    """sdpa_bwd_noalloc(): sdpa_bwd_ex on contiguous bf16 tensors with the library's static device
    scratch as the workspace (no allocation; SdpaBwdError with SCRATCH_TOO_SMALL when the problem
    needs more than NOALLOC_SCRATCH_BYTES)."""
    dims = _dims(q, k, v)
    _check(_load().sdpa_bwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
        *dims, -1.0 if scale is None else float(scale), int(causal), int(window_left),
        int(deterministic), _ptr(seq_q_lens), _ptr(seq_kv_lens), int(causal_bottom_right),
        int(window_right), _stream_handle(stream)))


def _bias_dtype(bias, q):
    import torch
    if bias is None:
        return _io_dtype(q)
    return FP32 if bias.dtype == torch.float32 else FP16 if bias.dtype == torch.float16 else BF16


def run_args(q, k, v, o, do, lse, dq, dk, dv, scale=None, causal=False, window_left=-1,
             deterministic=False, seq_q_lens=None, seq_kv_lens=None, causal_bottom_right=False,
             window_right=0, sink=None, dsink=None, bias=None, dbias=None, workspace=None,
             stream=None, events=None):
    """The sdpa_bwd_args struct of one call (tensors marshalled to device pointers)."""
    B, Hq, Hkv, Sq, Skv, Dqk, Dv = _dims(q, k, v)
    tensors = (q, k, v, o, do, dq, dk, dv)
    lay = _layouts(tensors)
    handles = None
    if events is not None:
        handles = (ctypes.c_void_p * 5)(
            *[ctypes.c_void_p(None if e is None else e.cuda_event) for e in events])
    a = Args()
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dO", do), ("lse", lse), ("dq", dq),
                 ("dk", dk), ("dv", dv), ("seq_q_lens", seq_q_lens), ("seq_kv_lens", seq_kv_lens),
                 ("sink", sink), ("dsink", dsink), ("workspace", workspace)):
        setattr(a, n, None if t is None else t.data_ptr())
    a.B, a.Hq, a.Hkv, a.Sq, a.Skv, a.Dqk, a.Dv = B, Hq, Hkv, Sq, Skv, Dqk, Dv
    a.scale = -1.0 if scale is None else float(scale)
    a.causal, a.causal_bottom_right = int(causal), int(causal_bottom_right)
    a.window_left, a.window_right = int(window_left), int(window_right)
    a.deterministic = int(deterministic)
    a.layouts = ctypes.cast(lay, ctypes.c_void_p).value
    a.dtype = _io_dtype(q)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.stream = None if stream is False else _stream_handle(stream).value
    a.events = None if handles is None else ctypes.cast(handles, ctypes.c_void_p).value
    a.bias = None if bias is None else bias.data_ptr()
    a.bias_dtype = _bias_dtype(bias, q)
    a.bias_batch = 1 if bias is None else int(bias.shape[0])
    a.dbias = None if dbias is None else dbias.data_ptr()
    # an io-type dBias (bf16 / fp16 tensor) is accumulated in fp32 and cast by dbias_cvt
    a.dbias_io = 0 if dbias is None or _bias_dtype(dbias, q) == FP32 else 1
    if a.dbias_io and dbias.dtype != q.dtype:
        raise ValueError("dbias must be float32 or of q's dtype")
    # keep the pointed-to ctypes arrays alive with the struct
    a._keep = (lay, handles)
    return a


def run_workspace_size(q, k, v, **kw) -> int:
    """sdpa_bwd_run_workspace_size() for a call on these q, k, v and keyword arguments (the other
    tensors' pointers, the workspace and the stream are not read)."""
    a = run_args(q, k, v, q, q, None, q, k, v, stream=False, **kw)
    return int(_load().sdpa_bwd_run_workspace_size(ctypes.byref(a)))


def run_dq_route(q, k, v, **kw) -> int:
    """sdpa_bwd_run_dq_route() for a call on these q, k, v and keyword arguments."""
    a = run_args(q, k, v, q, q, None, q, k, v, stream=False, **kw)
    return int(_load().sdpa_bwd_run_dq_route(ctypes.byref(a)))


def sdpa_bwd_run(q, k, v, o, do, lse, dq, dk, dv, scale=None, causal=False, window_left=-1,
                 deterministic=False, seq_q_lens=None, seq_kv_lens=None,
                 causal_bottom_right=False, window_right=0, sink=None, dsink=None, bias=None,
                 dbias=None, workspace=None, stream=None, events=None):
    """sdpa_bwd_run(): the superset entry point (any dense layout with a contiguous head dim,
    bf16 or fp16; the sink gradient: dsink (Hq,) fp32 is written when given, from the sink
    (Hq,) fp32 logits; an additive bias (1 or B, Hq, Sq, Skv) of the io type or fp32, with its
    gradient dbias when given: fp32, or of the io type (then accumulated in fp32 in the workspace
    and cast once)).  `workspace` must hold run_workspace_size(...) bytes."""
    a = run_args(q, k, v, o, do, lse, dq, dk, dv, scale, causal, window_left, deterministic,
                 seq_q_lens, seq_kv_lens, causal_bottom_right, window_right, sink, dsink, bias,
                 dbias, workspace, stream, events)
    _check(_load().sdpa_bwd_run(ctypes.byref(a)))


def nvfp4_qat_workspace_size(B, H, Sq, Skv, D=128, causal=False, deterministic=0) -> int:
    """sdpa_bwd_nvfp4_qat_workspace_size()."""
    return int(_load().sdpa_bwd_nvfp4_qat_workspace_size(int(B), int(H), int(Sq), int(Skv), int(D),
                                                         int(bool(causal)), int(deterministic)))


def sdpa_bwd_nvfp4_qat(q, k, v, o_hp, do, lse, dq, dk, dv, scale=None, causal=False,
                       deterministic=0, workspace=None, stream=None, events=None):
    """sdpa_bwd_nvfp4_qat(): the NVFP4 attention-QAT backward on contiguous (B, H, S, 128) bf16
    tensors; `workspace` must hold nvfp4_qat_workspace_size(...) bytes."""
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_load().sdpa_bwd_nvfp4_qat(_ptr(q), _ptr(k), _ptr(v), _ptr(o_hp), _ptr(do), _ptr(lse),
                                      _ptr(dq), _ptr(dk), _ptr(dv), B, H, Sq, Skv, D,
                                      0.0 if scale is None else float(scale), int(bool(causal)),
                                      int(deterministic), _ptr(workspace), ws_bytes,
                                      _stream_handle(stream), _events(events)))


def sdpa_bwd_preprocess(o, do, lse, stats, dq_accum=None, seq_q_lens=None, Dqk=0, stream=None):
    """sdpa_bwd_preprocess(): stats rows [LSE * log2 e, rowsum(O * dO)] (and zero dq_accum)."""
    B, Hq, Sq, Dv = o.shape
    _check(_load().sdpa_bwd_preprocess(_ptr(o), _ptr(do), _ptr(lse), _ptr(stats), _ptr(dq_accum),
                                       _ptr(seq_q_lens), B, Hq, Sq, Dv, int(Dqk),
                                       _stream_handle(stream)))


def attention_backward(q, k, v, o, do, lse, scale=None, causal=False, window_left=-1,
                       deterministic=False, seq_q_lens=None, seq_kv_lens=None,
                       causal_bottom_right=False, window_right=0, stream=None):
    """Allocate dq/dk/dv and the workspace with torch, then run sdpa_bwd_ex; returns (dq, dk, dv).

    The chain is enqueued on `stream` (default: torch's current stream), and dq, dk, dv are
    written there.  The caller orders the producers of the inputs before `stream`.  When `stream`
    is not the current stream, the workspace and the outputs are recorded on it, so torch's
    caching allocator does not hand their memory to another allocation before the chain is done
    with it."""
    import torch
    B, Hq, Hkv, Sq, Skv, Dqk, Dv = _dims(q, k, v)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    n = workspace_size(B, Hq, Hkv, Sq, Skv, Dqk, Dv, causal, window_left, deterministic,
                       seq_q_lens is not None)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)
    sdpa_bwd_ex(q, k, v, o, do, lse, dq, dk, dv, scale, causal, window_left, deterministic,
                seq_q_lens, seq_kv_lens, causal_bottom_right, window_right, ws, stream)
    if stream is not None and stream != torch.cuda.current_stream(q.device):
        for t in (ws, dq, dk, dv):
            t.record_stream(stream)
    return dq, dk, dv
