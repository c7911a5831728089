"""Python binding of libpa_verify.so — paged verify attention on MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/pa_verify.h).  torch provides device
memory and the current stream.  Importing this module loads nothing; the
first call loads the in-tree library and raises if it is missing — there is
no fallback.

Functions keep the C names:
  pa_verify_forward(q, k_cache, v_cache, block_tables, past_lens,
                    subsequence_begins, max_context_len, scale, out=None, ...)
  pa_verify_forward_u8(q, k_cache, v_cache, k_scale_zp, v_scale_zp, ...)
  pa_verify_forward_noalloc(q, ..., out, ...)  (static scratch, no workspace)
  pa_verify_workspace_bytes(...), pa_verify_make_plan(...),
  pa_verify_read_status(...), pa_verify_status_string(code)
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpa_verify.so")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP, PA_ERR_DEVICE_CONTRACT = range(6)
PA_F16, PA_BF16, PA_U8 = 0, 1, 2
PA_PAGES_TILED, PA_PAGES_ROW_MAJOR = 0, 1

# every symbol include/pa_verify.h declares
EXPORTS = ("pa_verify_make_plan", "pa_verify_workspace_bytes", "pa_verify_forward",
           "pa_verify_forward_noalloc", "pa_verify_forward_u8", "pa_kv_append", "pa_kv_append_u8",
           "pa_verify_read_status", "pa_verify_status_string")
# bytes of the static device scratch pa_verify_forward_noalloc works in
NOALLOC_SCRATCH_BYTES = 32 << 20


class PaVerifyParams(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
        ("sliding_window", ctypes.c_int32), ("num_segments", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("max_query_len", ctypes.c_int32),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("prof_event_begin", ctypes.c_void_p), ("prof_event_end", ctypes.c_void_p),
        ("tree_mask", ctypes.c_void_p),
        ("page_layout", ctypes.c_int32),
    ]


class PaVerifyPlan(ctypes.Structure):
    _fields_ = [
        ("num_segments", ctypes.c_int32), ("steps_per_segment", ctypes.c_int32),
        ("num_steps", ctypes.c_int32), ("row_blocks", ctypes.c_int32),
        ("worklist", ctypes.c_int32), ("target_items", ctypes.c_int32),
        ("keys_per_step", ctypes.c_int32), ("span", ctypes.c_int32),
        ("waves_per_group", ctypes.c_int32), ("max_steps_per_segment", ctypes.c_int32),
        ("grid", ctypes.c_int32 * 3),
        ("block_threads", ctypes.c_int32), ("combine_grid", ctypes.c_int32 * 3),
        ("combine_threads", ctypes.c_int32), ("workspace_bytes", ctypes.c_size_t),
        ("direct", ctypes.c_int32), ("small_groups", ctypes.c_int32),
    ]

    def as_dict(self):
        return {f: (list(getattr(self, f)) if f.endswith("grid") else getattr(self, f))
                for f, _ in self._fields_}


class PaVerifyError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(pa_verify_status_string(code))
        self.code = code


_lib = None
_lock = threading.Lock()


def lib():
    """The loaded libpa_verify.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise ImportError(f"{LIB_PATH} is missing: build it with "
                                      "`python -m speculative_decoding_verify_paged_amd.build`")
                L = ctypes.CDLL(LIB_PATH)
                vp, i32, P = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(PaVerifyParams)
                L.pa_verify_make_plan.argtypes = [P, i32, i32, ctypes.POINTER(PaVerifyPlan)]
                L.pa_verify_make_plan.restype = ctypes.c_int
                L.pa_verify_workspace_bytes.argtypes = [P, i32]
                L.pa_verify_workspace_bytes.restype = ctypes.c_size_t
                L.pa_verify_forward.argtypes = [vp, vp, vp, vp, vp, vp, i32, ctypes.c_float, vp, P]
                L.pa_verify_forward.restype = ctypes.c_int
                L.pa_verify_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, ctypes.c_float,
                                                        vp, P]
                L.pa_verify_forward_noalloc.restype = ctypes.c_int
                L.pa_verify_forward_u8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32,
                                                   ctypes.c_float, vp, P]
                L.pa_verify_forward_u8.restype = ctypes.c_int
                L.pa_kv_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, P]
                L.pa_kv_append.restype = ctypes.c_int
                L.pa_kv_append_u8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, P]
                L.pa_kv_append_u8.restype = ctypes.c_int
                L.pa_verify_read_status.argtypes = [P, ctypes.POINTER(i32)]
                L.pa_verify_read_status.restype = ctypes.c_int
                L.pa_verify_status_string.argtypes = [ctypes.c_int]
                L.pa_verify_status_string.restype = ctypes.c_char_p
                _lib = L
    return _lib


def pa_verify_status_string(code: int) -> str:
    return lib().pa_verify_status_string(int(code)).decode()


def make_params(*, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, block_size,
                num_blocks, max_blocks_per_seq, q_dtype, kv_dtype, sliding_window=0,
                num_segments=0, max_query_len=0, workspace=0, workspace_bytes=0, stream=0,
                prof_event_begin=0, prof_event_end=0, tree_mask=0,
                page_layout=PA_PAGES_TILED) -> PaVerifyParams:
    return PaVerifyParams(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, block_size,
                          num_blocks, max_blocks_per_seq, sliding_window, num_segments,
                          q_dtype, kv_dtype, max_query_len, workspace or None, workspace_bytes,
                          stream or None, prof_event_begin or None, prof_event_end or None,
                          tree_mask or None, page_layout)


def pa_verify_make_plan(params: PaVerifyParams, max_context_len: int, num_cus: int) -> dict:
    plan = PaVerifyPlan()
    rc = lib().pa_verify_make_plan(ctypes.byref(params), int(max_context_len), int(num_cus),
                                   ctypes.byref(plan))
    if rc != PA_OK:
        raise PaVerifyError(rc)
    return plan.as_dict()


def pa_verify_workspace_bytes(params: PaVerifyParams, max_context_len: int) -> int:
    return int(lib().pa_verify_workspace_bytes(ctypes.byref(params), int(max_context_len)))


# ---------------------------------------------------------------------------
# torch-facing calls
# ---------------------------------------------------------------------------
_ws_cache = {}
# Workspaces the cached one replaced, kept allocated until the process ends: a
# HIP graph captured before a growth still holds their pointers and writes its
# partials and status word there on every replay.
_ws_retired = {}


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return PA_F16
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype == torch.uint8:
        return PA_U8
    raise ValueError(f"unsupported dtype {t.dtype}")


def workspace(nbytes: int, device):
    """A zero-initialised device workspace of at least nbytes, cached per device.

    Every call on the device that is given no ``workspace=`` uses this one
    buffer, so such calls must be ordered (one stream, or streams that wait
    on each other); calls that may run concurrently need their own
    workspaces.  Allocating or growing it synchronises the device (no call
    still uses the old buffer, and the zeroed status word is in place before
    any stream runs on the new one), so it cannot happen during graph capture:
    make one eager call with the largest shape first.  Growth at least doubles
    the buffer, and a replaced buffer stays allocated (a graph captured
    earlier keeps using it; ``pa_verify_read_status`` reads its status word
    too), so the memory held is at most twice the largest need."""
    torch = _torch()
    key = (str(device),)
    old = _ws_cache.get(key)
    if old is None or old.numel() < nbytes:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("the cached workspace must be sized before graph capture: make one "
                               "eager call with the largest shape first, or pass workspace=")
        torch.cuda.synchronize(device)
        size = max(nbytes, 1 << 20, 0 if old is None else 2 * old.numel())
        buf = torch.zeros(size, dtype=torch.uint8, device=device)
        if old is not None:
            _ws_retired.setdefault(key, []).append(old)
        torch.cuda.synchronize(device)
        _ws_cache[key] = buf
        return buf
    return old


def _check(t, name, dtype=None, ndim=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


class PreparedCall:
    """One forward call with its arguments checked and marshalled once.
    Calling it enqueues the call again with the same pointers and sizes;
    only the stream and the profiling events may change.  The tensors it was
    prepared from must stay alive and unmoved."""

    def __init__(self, fn, args, params, out, keep):
        self._fn, self._args, self._params, self.out = fn, args, params, out
        self._pref = ctypes.byref(params)
        self._keep = keep

    def __call__(self, stream: Optional[int] = None, prof_events=None):
        p = self._params
        if stream is not None:
            p.stream = stream or None
        p.prof_event_begin, p.prof_event_end = prof_events if prof_events else (None, None)
        rc = self._fn(*self._args, self._pref)
        if rc != PA_OK:
            raise PaVerifyError(rc)
        return self.out


def _call(u8, q, k_cache, v_cache, k_scale_zp, v_scale_zp, block_tables, past_lens,
          subsequence_begins, max_context_len, scale, out, sliding_window, num_segments,
          ws, stream, prof_events, prepare=False, max_query_len=0, tree_mask=None,
          noalloc=False, page_layout=PA_PAGES_TILED):
    torch = _torch()
    dev = q.device
    _check(q, "q", ndim=3, device=dev)
    _check(k_cache, "k_cache", ndim=4, device=dev)
    _check(v_cache, "v_cache", ndim=4, device=dev)
    for n, t in (("block_tables", block_tables), ("past_lens", past_lens),
                 ("subsequence_begins", subsequence_begins)):
        _check(t, n, dtype=torch.int32, device=dev)
    num_tokens, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != (nb, Hkv, bs, D):
        raise ValueError("k_cache and v_cache must both be [nb, Hkv, bs, D] (page contents in "
                         "the order page_layout names, see include/pa_verify.h)")
    if k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache dtypes differ")
    if u8:
        for n, t in (("k_scale_zp", k_scale_zp), ("v_scale_zp", v_scale_zp)):
            _check(t, n, dtype=torch.float16, device=dev)
            if tuple(t.shape) != (nb, Hkv, bs, 2):
                raise ValueError(f"{n} must be [nb, Hkv, bs, 2] float16")
    if block_tables.dim() != 2 or past_lens.dim() != 1 or subsequence_begins.dim() != 1:
        raise ValueError("block_tables must be 2-D, past_lens and subsequence_begins 1-D")
    num_seqs = past_lens.shape[0]
    if block_tables.shape[0] != num_seqs or subsequence_begins.shape[0] != num_seqs + 1:
        raise ValueError("block_tables / subsequence_begins do not match past_lens")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", dtype=q.dtype, device=dev)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    if tree_mask is not None:
        _check(tree_mask, "tree_mask", ndim=1, device=dev)
        if tree_mask.dtype not in (torch.int32, torch.uint32) or tree_mask.shape[0] != num_tokens:
            raise ValueError("tree_mask must be a 32-bit integer tensor of num_tokens words")
    params = make_params(num_seqs=num_seqs, num_tokens=num_tokens, num_q_heads=Hq,
                         num_kv_heads=Hkv, head_dim=D, block_size=bs, num_blocks=nb,
                         max_blocks_per_seq=block_tables.shape[1], q_dtype=_dtype_code(q),
                         kv_dtype=_dtype_code(k_cache), sliding_window=int(sliding_window),
                         num_segments=int(num_segments), max_query_len=int(max_query_len),
                         tree_mask=0 if tree_mask is None else tree_mask.data_ptr(),
                         page_layout=int(page_layout))
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    params.stream = stream or None
    if noalloc:
        if ws is not None:
            raise ValueError("the no-allocation call works in the library's static scratch: "
                             "pass no workspace")
    else:
        need = pa_verify_workspace_bytes(params, max_context_len)
        if need == 0:
            # let the library name the problem
            need = 256
        if ws is None:
            with torch.cuda.device(dev):
                ws = workspace(need, dev)
        else:
            _check(ws, "workspace", dtype=torch.uint8, ndim=1, device=dev)
        params.workspace = ws.data_ptr()
        params.workspace_bytes = ws.numel() * ws.element_size()
    if prof_events is not None:
        params.prof_event_begin = prof_events[0]
        params.prof_event_end = prof_events[1]
    L = lib()
    if u8:
        fn = L.pa_verify_forward_u8
        args = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), k_scale_zp.data_ptr(),
                v_scale_zp.data_ptr(), block_tables.data_ptr(), past_lens.data_ptr(),
                subsequence_begins.data_ptr(), int(max_context_len), float(scale), out.data_ptr())
    else:
        fn = L.pa_verify_forward_noalloc if noalloc else L.pa_verify_forward
        args = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
                past_lens.data_ptr(), subsequence_begins.data_ptr(), int(max_context_len),
                float(scale), out.data_ptr())
    if prepare:
        keep = (q, k_cache, v_cache, k_scale_zp, v_scale_zp, block_tables, past_lens,
                subsequence_begins, out, ws, tree_mask)
        return PreparedCall(fn, args, params, out, keep)
    rc = fn(*args, ctypes.byref(params))
    if rc != PA_OK:
        raise PaVerifyError(rc)
    return out


def pa_verify_forward(q, k_cache, v_cache, block_tables, past_lens, subsequence_begins,
                      max_context_len: int, scale: float, out=None, *, sliding_window: int = 0,
                      num_segments: int = 0, workspace=None, stream: Optional[int] = None,
                      prof_events=None, max_query_len: int = 0, tree_mask=None,
        page_layout: int = PA_PAGES_TILED):
    """Paged verify attention over an f16/bf16 cache; returns ``out``.

    q [num_tokens, Hq, D]; k_cache, v_cache [nb, Hkv, bs, D] with each page's
    bs * D elements in the tiled order the C header defines;
    block_tables [num_seqs, max_blocks_per_seq], past_lens [num_seqs],
    subsequence_begins [num_seqs + 1] (int32, device).  ``stream`` is a raw
    hipStream_t (default: torch's current stream); ``prof_events`` is an
    optional pair of raw hipEvent_t recorded around the segment kernel.
    ``max_query_len`` bounds the new tokens per sequence (0: derived from
    num_tokens and num_seqs); ``tree_mask`` is an optional int32/uint32
    device tensor [num_tokens] of draft-tree visibility words.
    ``workspace``: a device uint8 tensor of at least pa_verify_workspace_bytes,
    its first 4 bytes zeroed once; default the per-device cached one (see
    ``workspace()``: calls that share it must be ordered)."""
    return _call(False, q, k_cache, v_cache, None, None, block_tables, past_lens,
                 subsequence_begins, max_context_len, scale, out, sliding_window, num_segments,
                 workspace, stream, prof_events, max_query_len=max_query_len, tree_mask=tree_mask,
                 page_layout=page_layout)


def pa_verify_forward_noalloc(q, k_cache, v_cache, block_tables, past_lens, subsequence_begins,
                              max_context_len: int, scale: float, out, *, sliding_window: int = 0,
                              num_segments: int = 0, stream: Optional[int] = None,
                              max_query_len: int = 0, tree_mask=None,
        page_layout: int = PA_PAGES_TILED):
    """pa_verify_forward without any workspace: the library works in its static
    device scratch (32 MiB per GPU), so nothing is allocated by the call or
    here — ``out`` must be given.  Calls on one GPU share that scratch and
    must not overlap; a contract violation shows only as NaN rows."""
    if out is None:
        raise ValueError("pass out: the no-allocation call allocates nothing")
    return _call(False, q, k_cache, v_cache, None, None, block_tables, past_lens,
                 subsequence_begins, max_context_len, scale, out, sliding_window, num_segments,
                 None, stream, None, max_query_len=max_query_len, tree_mask=tree_mask,
                 noalloc=True, page_layout=page_layout)


def pa_verify_forward_u8(q, k_cache, v_cache, k_scale_zp, v_scale_zp, block_tables, past_lens,
                         subsequence_begins, max_context_len: int, scale: float, out=None, *,
                         sliding_window: int = 0, num_segments: int = 0, workspace=None,
                         stream: Optional[int] = None, prof_events=None, max_query_len: int = 0,
                         tree_mask=None,
        page_layout: int = PA_PAGES_TILED):
    """The same over a u8 cache with f16 (scale, zero point) per token per KV head."""
    return _call(True, q, k_cache, v_cache, k_scale_zp, v_scale_zp, block_tables, past_lens,
                 subsequence_begins, max_context_len, scale, out, sliding_window, num_segments,
                 workspace, stream, prof_events, max_query_len=max_query_len, tree_mask=tree_mask,
                 page_layout=page_layout)


def pa_verify_read_status(device=None) -> int:
    """Synchronise and read-and-clear the sticky device status word of the
    cached workspace and of the workspaces it replaced (graphs captured
    before a growth still write there); PA_ERR_DEVICE_CONTRACT if any was set."""
    torch = _torch()
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    key = (str(dev),)
    bufs = list(_ws_retired.get(key, [])) + ([_ws_cache[key]] if key in _ws_cache else [])
    result = PA_OK
    for buf in bufs:
        p = PaVerifyParams()
        p.workspace = buf.data_ptr()
        p.workspace_bytes = buf.numel()
        p.stream = torch.cuda.current_stream(dev).cuda_stream or None
        st = ctypes.c_int32(0)
        rc = lib().pa_verify_read_status(ctypes.byref(p), ctypes.byref(st))
        if rc != PA_OK:
            raise PaVerifyError(rc)
        if st.value != PA_OK:
            result = int(st.value)
    return result


def prepare_forward(q, k_cache, v_cache, block_tables, past_lens, subsequence_begins,
                    max_context_len: int, scale: float, out=None, *, sliding_window: int = 0,
                    num_segments: int = 0, workspace=None, stream: Optional[int] = None,
                    max_query_len: int = 0, tree_mask=None,
        page_layout: int = PA_PAGES_TILED):
    """pa_verify_forward's checks and marshalling done once: returns a
    PreparedCall that enqueues the same call each time it is called."""
    return _call(False, q, k_cache, v_cache, None, None, block_tables, past_lens,
                 subsequence_begins, max_context_len, scale, out, sliding_window, num_segments,
                 workspace, stream, None, prepare=True, max_query_len=max_query_len,
                 tree_mask=tree_mask, page_layout=page_layout)


def prepare_forward_u8(q, k_cache, v_cache, k_scale_zp, v_scale_zp, block_tables, past_lens,
                       subsequence_begins, max_context_len: int, scale: float, out=None, *,
                       sliding_window: int = 0, num_segments: int = 0, workspace=None,
                       stream: Optional[int] = None, max_query_len: int = 0, tree_mask=None,
        page_layout: int = PA_PAGES_TILED):
    """pa_verify_forward_u8's checks and marshalling done once (see prepare_forward)."""
    return _call(True, q, k_cache, v_cache, k_scale_zp, v_scale_zp, block_tables, past_lens,
                 subsequence_begins, max_context_len, scale, out, sliding_window, num_segments,
                 workspace, stream, None, prepare=True, max_query_len=max_query_len,
                 tree_mask=tree_mask, page_layout=page_layout)


def _append(u8, k_new, v_new, k_cache, v_cache, k_scale_zp, v_scale_zp, block_tables, past_lens,
            subsequence_begins, max_query_len, stream, page_layout=PA_PAGES_TILED):
    torch = _torch()
    dev = k_new.device
    _check(k_new, "k_new", ndim=3, device=dev)
    _check(v_new, "v_new", ndim=3, device=dev)
    if v_new.shape != k_new.shape or v_new.dtype != k_new.dtype:
        raise ValueError("k_new and v_new must have the same shape and dtype")
    _check(k_cache, "k_cache", ndim=4, device=dev)
    _check(v_cache, "v_cache", ndim=4, device=dev)
    for n, t in (("block_tables", block_tables), ("past_lens", past_lens),
                 ("subsequence_begins", subsequence_begins)):
        _check(t, n, dtype=torch.int32, device=dev)
    num_tokens, Hkv, D = k_new.shape
    nb, Hkv2, bs, D2 = k_cache.shape
    if (Hkv2, D2) != (Hkv, D) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("caches must be [nb, Hkv, bs, D] matching k_new's Hkv and D")
    if u8:
        for n, t in (("k_scale_zp", k_scale_zp), ("v_scale_zp", v_scale_zp)):
            _check(t, n, dtype=torch.float16, device=dev)
            if tuple(t.shape) != (nb, Hkv, bs, 2):
                raise ValueError(f"{n} must be [nb, Hkv, bs, 2] float16")
    num_seqs = past_lens.shape[0]
    if block_tables.shape[0] != num_seqs or subsequence_begins.shape[0] != num_seqs + 1:
        raise ValueError("block_tables / subsequence_begins do not match past_lens")
    params = make_params(num_seqs=num_seqs, num_tokens=num_tokens, num_q_heads=Hkv,
                         num_kv_heads=Hkv, head_dim=D, block_size=bs, num_blocks=nb,
                         max_blocks_per_seq=block_tables.shape[1], q_dtype=_dtype_code(k_new),
                         kv_dtype=_dtype_code(k_cache), max_query_len=int(max_query_len),
                         page_layout=int(page_layout))
    params.stream = (torch.cuda.current_stream(dev).cuda_stream if stream is None else stream) or None
    with torch.cuda.device(dev):
        ws = workspace(256, dev)
    params.workspace = ws.data_ptr()
    params.workspace_bytes = ws.numel()
    L = lib()
    if u8:
        rc = L.pa_kv_append_u8(k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
                               v_cache.data_ptr(), k_scale_zp.data_ptr(), v_scale_zp.data_ptr(),
                               block_tables.data_ptr(), past_lens.data_ptr(),
                               subsequence_begins.data_ptr(), ctypes.byref(params))
    else:
        rc = L.pa_kv_append(k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
                            v_cache.data_ptr(), block_tables.data_ptr(), past_lens.data_ptr(),
                            subsequence_begins.data_ptr(), ctypes.byref(params))
    if rc != PA_OK:
        raise PaVerifyError(rc)


def pa_kv_append(k_new, v_new, k_cache, v_cache, block_tables, past_lens, subsequence_begins, *,
                 max_query_len: int = 0, stream: Optional[int] = None,
                 page_layout: int = PA_PAGES_TILED):
    """Write the new tokens' K/V ([num_tokens, Hkv, D], f16 or bf16) into an
    f16/bf16 cache of the same dtype at positions past_len + i (in place)."""
    _append(False, k_new, v_new, k_cache, v_cache, None, None, block_tables, past_lens,
            subsequence_begins, max_query_len, stream, page_layout)


def pa_kv_append_u8(k_new, v_new, k_cache, v_cache, k_scale_zp, v_scale_zp, block_tables,
                    past_lens, subsequence_begins, *, max_query_len: int = 0,
                    stream: Optional[int] = None, page_layout: int = PA_PAGES_TILED):
    """The same into a u8 cache: each (token, KV head) row is quantised and its
    f16 (scale, zero point) written to k_scale_zp / v_scale_zp (in place)."""
    _append(True, k_new, v_new, k_cache, v_cache, k_scale_zp, v_scale_zp, block_tables, past_lens,
            subsequence_begins, max_query_len, stream, page_layout)

