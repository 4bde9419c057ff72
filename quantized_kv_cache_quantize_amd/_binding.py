"""ctypes binding for libkvq.so: names mirror the C ABI in include/kvq.h."""

from __future__ import annotations

import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libkvq.so")

KVQ_F16, KVQ_F32 = 0, 1
KERNEL_AUTO, KERNEL_VALU, KERNEL_MFMA, KERNEL_MFMA_SPLIT, KERNEL_MFMA_WAVE = 0, 1, 2, 3, 4


class KvqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %s (%d)" % (fn, status_str(status), status))
        self.status = status


class _Cache(C.Structure):
    _fields_ = [
        ("k_q", C.c_void_p),
        ("v_q", C.c_void_p),
        ("k_scale", C.c_void_p),
        ("k_bias", C.c_void_p),
        ("v_scale", C.c_void_p),
        ("v_bias", C.c_void_p),
        ("batch", C.c_int32),
        ("kv_heads", C.c_int32),
        ("head_dim", C.c_int32),
        ("group", C.c_int32),
        ("capacity", C.c_int64),
        ("bits", C.c_int32),
    ]


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Load libkvq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libkvq.so not built: run __graft_entry__.build() or "
                          "python -m quantized_kv_cache_quantize_amd.build")
    L = C.CDLL(_LIB_PATH)
    vp, i32, i64, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_float
    cp = C.POINTER(_Cache)
    L.kvq_version.restype = C.c_char_p
    L.kvq_version.argtypes = []
    L.kvq_status_str.restype = C.c_char_p
    L.kvq_status_str.argtypes = [C.c_int]
    L.kvq_num_chunks.restype = i64
    L.kvq_num_chunks.argtypes = [i64, i32]
    L.kvq_cache_bytes.restype = i64
    L.kvq_cache_bytes.argtypes = [i32, i32, i32, i32, i64, i32]
    L.kvq_hbm_read.restype = C.c_int
    L.kvq_hbm_read.argtypes = [vp, i64, C.c_uint32, vp, vp]
    L.kvq_quantize_kv_append.restype = C.c_int
    L.kvq_quantize_kv_append.argtypes = [cp, i64, vp, vp, C.c_int, i64, vp]
    L.kvq_quantize_kv_append_rotated.restype = C.c_int
    L.kvq_quantize_kv_append_rotated.argtypes = [cp, i64, vp, vp, C.c_int, i64, vp]
    L.kvq_hadamard_rotate.restype = C.c_int
    L.kvq_hadamard_rotate.argtypes = [vp, C.c_int, i64, i32, vp, vp]
    L.kvq_sdpa_int4_partial.restype = C.c_int
    L.kvq_sdpa_int4_partial.argtypes = [cp, i64, vp, C.c_int, i32, f32, i32, vp, vp, vp, C.c_int, vp]
    L.kvq_sdpa_int4_partial_timed.restype = C.c_int
    L.kvq_sdpa_int4_partial_timed.argtypes = [cp, i64, vp, C.c_int, i32, f32, i32, vp, vp, vp, C.c_int, vp, vp, vp]
    L.kvq_sdpa_int4_reduce.restype = C.c_int
    L.kvq_sdpa_int4_reduce.argtypes = [vp, vp, vp, i32, i32, i32, i64, vp, vp]
    L.kvq_decode_step.restype = C.c_int
    L.kvq_decode_step.argtypes = [cp, i64, vp, vp, C.c_int, vp, C.c_int, i32, f32, i32, vp, vp, vp, vp, C.c_int, vp]
    L.kvq_decode_step_rotated.restype = C.c_int
    L.kvq_decode_step_rotated.argtypes = [cp, i64, vp, vp, C.c_int, vp, C.c_int, i32, f32, i32, vp, vp, vp, vp, C.c_int,
                                          vp]
    L.kvq_decode_step_timed.restype = C.c_int
    L.kvq_decode_step_timed.argtypes = [cp, i64, vp, vp, C.c_int, vp, C.c_int, i32, f32, i32, vp, vp, vp, vp, C.c_int,
                                        vp, vp, vp]
    L.kvq_decode_step_noalloc.restype = C.c_int
    L.kvq_decode_step_noalloc.argtypes = [cp, i64, vp, vp, C.c_int, vp, C.c_int, i32, f32, i32, vp, C.c_int, vp]
    L.kvq_decode_workspace_bytes.restype = i64
    L.kvq_decode_workspace_bytes.argtypes = [cp, i32, i64]
    L.kvq_decode_step_single_launch.restype = C.c_int
    L.kvq_decode_step_single_launch.argtypes = [cp, i64, vp, vp, C.c_int, vp, C.c_int, i32, f32, vp, i64, vp, vp,
                                                vp, vp]
    L.kvq_sdpa_int4_prefill.restype = C.c_int
    L.kvq_sdpa_int4_prefill.argtypes = [cp, i64, i32, vp, C.c_int, i32, f32, vp, vp]
    L.kvq_sdpa_int4.restype = C.c_int
    L.kvq_sdpa_int4.argtypes = [cp, i64, vp, C.c_int, i32, f32, i32, vp, vp, vp, vp, C.c_int, vp]
    _lib = L
    return L


def version() -> str:
    return lib().kvq_version().decode()


def status_str(status: int) -> str:
    return lib().kvq_status_str(int(status)).decode()


def num_chunks(skv: int, chunk: int) -> int:
    return int(lib().kvq_num_chunks(int(skv), int(chunk)))


def cache_bytes(batch: int, kv_heads: int, head_dim: int, group: int, capacity: int, bits: int = 4) -> int:
    return int(lib().kvq_cache_bytes(batch, kv_heads, head_dim, group, capacity, bits))


def _check(fn: str, status: int):
    if status != 0:
        raise KvqError(fn, status)


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return KVQ_F16
    if t.dtype == torch.float32:
        return KVQ_F32
    return 99  # rejected by the library with KVQ_E_DTYPE


# ---- argument checks. The C ABI takes bare device pointers and cannot see
# sizes, so every tensor is checked here before anything is enqueued: shapes,
# dtypes and sizes of all arguments first (so that they are checked without a
# GPU too), then that each is a contiguous tensor on the cache's CUDA device.
# A failed check raises ValueError and nothing is launched.

def _fail(fn: str, msg: str):
    raise ValueError("%s: %s" % (fn, msg))


class _Args:
    """Checks of one call's tensors: need() checks a tensor's layout at once
    and keeps it; devices() then checks where all of them live."""

    def __init__(self, fn: str):
        self.fn = fn
        self.seen = []

    def need(self, name: str, t, shape=None, dtypes=None, min_numel=None):
        fn = self.fn
        if not isinstance(t, torch.Tensor):
            _fail(fn, "%s must be a torch.Tensor" % name)
        if shape is not None and tuple(t.shape) != tuple(shape):
            _fail(fn, "%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
        if dtypes is not None and t.dtype not in dtypes:
            _fail(fn, "%s has dtype %s, expected one of %s" % (name, t.dtype, [str(d) for d in dtypes]))
        if min_numel is not None and t.numel() < min_numel:
            _fail(fn, "%s holds %d elements, needs at least %d" % (name, t.numel(), min_numel))
        if not t.is_contiguous():
            _fail(fn, "%s must be contiguous" % name)
        self.seen.append((name, t))
        return t

    def devices(self, device=None):
        for name, t in self.seen:
            if t.device.type != "cuda":
                _fail(self.fn, "%s must be a CUDA (HIP) device tensor, got %s" % (name, t.device))
            if device is not None and t.device != device:
                _fail(self.fn, "%s is on %s, the cache is on %s" % (name, t.device, device))


_FP = (torch.float16, torch.float32)
_F32 = (torch.float32,)


def _rows_arg(A: _Args, name: str, t, cache, allow_3d: bool):
    """k_new / v_new: [B][Hkv][n][D] (or [B][Hkv][D] for one row where
    allow_3d); returns n."""
    B, H, D = cache.batch, cache.kv_heads, cache.head_dim
    if not isinstance(t, torch.Tensor):
        _fail(A.fn, "%s must be a torch.Tensor" % name)
    if t.dim() == 3 and allow_3d:
        A.need(name, t, (B, H, D), _FP)
        return 1
    if t.dim() != 4 or tuple(t.shape[:2]) != (B, H) or t.shape[3] != D or (allow_3d and t.shape[2] != 1):
        want = "[%d, %d, %s, %d]" % (B, H, "1" if allow_3d else "n", D)
        if allow_3d:
            want += " or [%d, %d, %d]" % (B, H, D)
        _fail(A.fn, "%s has shape %s, expected %s" % (name, tuple(t.shape), want))
    A.need(name, t, None, _FP)
    return int(t.shape[2])


def _query_arg(A: _Args, q, cache, dims: int = 3):
    if not isinstance(q, torch.Tensor) or q.dim() != dims:
        _fail(A.fn, "q must be a %d-D tensor" % dims)
    B, Hq, D = q.shape[0], q.shape[1], q.shape[-1]
    if B != cache.batch or D != cache.head_dim or Hq < 1 or Hq % cache.kv_heads:
        _fail(A.fn, "q has shape %s: batch %d, head_dim %d and a multiple of %d query heads expected" % (
            tuple(q.shape), cache.batch, cache.head_dim, cache.kv_heads))
    A.need("q", q, None, _FP)
    return B, Hq, D


def _workspace_arg(A: _Args, ws, B, Hq, D, C):
    if ws is None or len(ws) != 3:
        _fail(A.fn, "workspace must be (part_m, part_l, part_acc)")
    m, l, acc = ws
    A.need("part_m", m, None, _F32, B * Hq * C)
    A.need("part_l", l, None, _F32, B * Hq * C)
    A.need("part_acc", acc, None, _F32, B * Hq * C * D)
    return m, l, acc


class QuantKVCache:
    """One layer's quantised cache in device memory (allocated by PyTorch).

    k_q, v_q: int32 tensors [B][Hkv][cap][D*bits/32] holding the uint32 words
    (bits = 4: eight nibbles per word; bits = 8: four bytes per word);
    k_scale, k_bias, v_scale, v_bias: float16 [B][Hkv][cap][D/G]."""

    def __init__(self, batch: int, kv_heads: int, head_dim: int, capacity: int, group: int = 64,
                 device="cuda", tensors=None, bits: int = 4):
        self.batch, self.kv_heads, self.head_dim = batch, kv_heads, head_dim
        self.capacity, self.group, self.bits = capacity, group, bits
        if bits not in (4, 8) or head_dim % 8 or group < 1 or head_dim % group:
            _fail("QuantKVCache", "unsupported layout (head_dim %d, group %d, bits %d)" % (head_dim, group, bits))
        wshape = (batch, kv_heads, capacity, head_dim * bits // 32)
        sshape = (batch, kv_heads, capacity, head_dim // group)
        if tensors is not None:
            self.k_q, self.v_q, self.k_scale, self.k_bias, self.v_scale, self.v_bias = tensors
            A = _Args("QuantKVCache")
            for name in ("k_q", "v_q"):
                A.need(name, getattr(self, name), wshape, (torch.int32,))
            for name in ("k_scale", "k_bias", "v_scale", "v_bias"):
                A.need(name, getattr(self, name), sshape, (torch.float16,))
            A.devices(self.k_q.device)
        else:
            self.k_q = torch.zeros(wshape, dtype=torch.int32, device=device)
            self.v_q = torch.zeros(wshape, dtype=torch.int32, device=device)
            self.k_scale = torch.zeros(sshape, dtype=torch.float16, device=device)
            self.k_bias = torch.zeros(sshape, dtype=torch.float16, device=device)
            self.v_scale = torch.zeros(sshape, dtype=torch.float16, device=device)
            self.v_bias = torch.zeros(sshape, dtype=torch.float16, device=device)

    @property
    def device(self):
        return self.k_q.device

    def c_struct(self) -> _Cache:
        return _Cache(_ptr(self.k_q), _ptr(self.v_q), _ptr(self.k_scale), _ptr(self.k_bias), _ptr(self.v_scale),
                      _ptr(self.v_bias), self.batch, self.kv_heads, self.head_dim, self.group, self.capacity,
                      self.bits)

    def nbytes(self) -> int:
        return cache_bytes(self.batch, self.kv_heads, self.head_dim, self.group, self.capacity, self.bits)

    def tensors(self):
        return (self.k_q, self.v_q, self.k_scale, self.k_bias, self.v_scale, self.v_bias)


Int4KVCache = QuantKVCache  # the int4 cache of the pages (bits=4, the default)


def _append_rows(fn, cache, k_new, v_new):
    A = _Args(fn)
    n = _rows_arg(A, "k_new", k_new, cache, allow_3d=False)
    if _rows_arg(A, "v_new", v_new, cache, allow_3d=False) != n or v_new.dtype != k_new.dtype:
        _fail(fn, "k_new and v_new must have the same shape and dtype")
    A.devices(cache.device)
    return n


def quantize_kv_append(cache: QuantKVCache, length: int, k_new: torch.Tensor, v_new: torch.Tensor,
                       stream=None) -> None:
    """kvq_quantize_kv_append: quantise k_new, v_new [B][Hkv][n][D] (fp16 or
    fp32, contiguous) into cache rows [length, length + n)."""
    n = _append_rows("quantize_kv_append", cache, k_new, v_new)
    cs = cache.c_struct()
    _check("kvq_quantize_kv_append",
           lib().kvq_quantize_kv_append(C.byref(cs), int(length), _ptr(k_new), _ptr(v_new), _dtype_code(k_new),
                                        int(n), _stream(stream)))


def quantize_kv_append_rotated(cache: QuantKVCache, length: int, k_new: torch.Tensor, v_new: torch.Tensor,
                               stream=None) -> None:
    """kvq_quantize_kv_append_rotated: Hadamard-rotate, then quantise, fp16
    rows k_new, v_new [B][Hkv][n][D] (contiguous) into cache rows
    [length, length + n)."""
    n = _append_rows("quantize_kv_append_rotated", cache, k_new, v_new)
    cs = cache.c_struct()
    _check("kvq_quantize_kv_append_rotated",
           lib().kvq_quantize_kv_append_rotated(C.byref(cs), int(length), _ptr(k_new), _ptr(v_new),
                                                _dtype_code(k_new), int(n), _stream(stream)))


def hadamard_rotate(x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """kvq_hadamard_rotate: rotate every row of x [..., D] (fp16 or fp32,
    contiguous) by H_D / sqrt(D); returns fp32 `out` (new, or the one given,
    which may be x itself when x is fp32)."""
    A = _Args("hadamard_rotate")
    if not isinstance(x, torch.Tensor) or x.dim() < 1:
        _fail(A.fn, "x must be a tensor [..., D]")
    A.need("x", x, None, _FP)
    d = x.shape[-1]
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    A.need("out", out, x.shape, _F32)
    A.devices(x.device)
    _check("kvq_hadamard_rotate",
           lib().kvq_hadamard_rotate(_ptr(x), _dtype_code(x), int(x.numel() // d), int(d), _ptr(out),
                                     _stream(stream)))
    return out


def hbm_read(buf: torch.Tensor, sink: torch.Tensor, key: int = 0xFFFFFFFF, stream=None) -> None:
    """kvq_hbm_read: read every byte of the contiguous device tensor `buf`
    once (a measurement helper); `sink` is a device int32 tensor of at least
    one element, written only when a thread's XOR of its words equals key."""
    A = _Args("hbm_read")
    A.need("buf", buf)
    A.need("sink", sink, None, (torch.int32,), 1)
    A.devices(buf.device)
    _check("kvq_hbm_read", lib().kvq_hbm_read(_ptr(buf), int(buf.numel() * buf.element_size()), int(key) & 0xFFFFFFFF,
                                              _ptr(sink), _stream(stream)))


def partials_buffers(batch: int, hq: int, head_dim: int, skv: int, chunk: int = 512, device="cuda"):
    """Allocate (part_m, part_l, part_acc) for the split-K workspace."""
    nc = num_chunks(skv, chunk)
    m = torch.empty((batch, hq, nc), dtype=torch.float32, device=device)
    l = torch.empty((batch, hq, nc), dtype=torch.float32, device=device)
    acc = torch.empty((batch, hq, nc, head_dim), dtype=torch.float32, device=device)
    return m, l, acc


def _partial_args(fn, cache, skv, q, chunk, ws):
    A = _Args(fn)
    B, Hq, D = _query_arg(A, q, cache)
    ws = _workspace_arg(A, ws, B, Hq, D, num_chunks(skv, chunk))
    A.devices(cache.device)
    return (Hq,) + ws


def sdpa_int4_partial(cache: QuantKVCache, skv: int, q: torch.Tensor, softmax_scale: float, chunk: int,
                      part_m: torch.Tensor, part_l: torch.Tensor, part_acc: torch.Tensor,
                      kernel: int = KERNEL_AUTO, stream=None) -> None:
    """kvq_sdpa_int4_partial: q [B][Hq][D] fp16/fp32 contiguous."""
    hq, m, l, acc = _partial_args("sdpa_int4_partial", cache, skv, q, chunk, (part_m, part_l, part_acc))
    cs = cache.c_struct()
    _check("kvq_sdpa_int4_partial",
           lib().kvq_sdpa_int4_partial(C.byref(cs), int(skv), _ptr(q), _dtype_code(q), hq,
                                       float(softmax_scale), int(chunk), _ptr(m), _ptr(l),
                                       _ptr(acc), int(kernel), _stream(stream)))


def _event_handle(ev) -> int:
    """Raw hipEvent_t of a torch.cuda.Event (created on first record)."""
    if ev.cuda_event == 0:
        ev.record()
    return ev.cuda_event


def sdpa_int4_partial_timed(cache: QuantKVCache, skv: int, q: torch.Tensor, softmax_scale: float, chunk: int,
                            part_m: torch.Tensor, part_l: torch.Tensor, part_acc: torch.Tensor, start, stop,
                            kernel: int = KERNEL_AUTO, stream=None) -> None:
    """kvq_sdpa_int4_partial_timed: as sdpa_int4_partial, with torch.cuda.Event
    start/stop (enable_timing=True) recorded at the kernel's own start and end."""
    hq, m, l, acc = _partial_args("sdpa_int4_partial_timed", cache, skv, q, chunk, (part_m, part_l, part_acc))
    cs = cache.c_struct()
    _check("kvq_sdpa_int4_partial_timed",
           lib().kvq_sdpa_int4_partial_timed(C.byref(cs), int(skv), _ptr(q), _dtype_code(q), hq,
                                             float(softmax_scale), int(chunk), _ptr(m), _ptr(l),
                                             _ptr(acc), int(kernel), _stream(stream), _event_handle(start),
                                             _event_handle(stop)))


def sdpa_int4_reduce(part_m: torch.Tensor, part_l: torch.Tensor, part_acc: torch.Tensor, out: torch.Tensor,
                     stream=None) -> None:
    """kvq_sdpa_int4_reduce: part_acc [B][Hq][C][D], part_m and part_l
    [B][Hq][C], out [B][Hq][D] fp32."""
    A = _Args("sdpa_int4_reduce")
    if not isinstance(part_acc, torch.Tensor) or part_acc.dim() != 4:
        _fail(A.fn, "part_acc must be a 4-D tensor [B][Hq][C][D]")
    b, hq, nc, d = part_acc.shape
    A.need("part_acc", part_acc, None, _F32)
    A.need("part_m", part_m, (b, hq, nc), _F32)
    A.need("part_l", part_l, (b, hq, nc), _F32)
    A.need("out", out, (b, hq, d), _F32)
    A.devices(part_acc.device)
    _check("kvq_sdpa_int4_reduce",
           lib().kvq_sdpa_int4_reduce(_ptr(part_m), _ptr(part_l), _ptr(part_acc), b, hq, d, nc, _ptr(out),
                                      _stream(stream)))


def _out_arg(A: _Args, out, B, Hq, D, device):
    if out is None:
        return torch.empty((B, Hq, D), dtype=torch.float32, device=device)
    return A.need("out", out, (B, Hq, D), _F32)


def sdpa_int4(cache: QuantKVCache, skv: int, q: torch.Tensor, softmax_scale: float, chunk: int = 512,
              out: torch.Tensor | None = None, workspace=None, kernel: int = KERNEL_AUTO, stream=None):
    """kvq_sdpa_int4: both phases on one stream; returns out [B][Hq][D] fp32."""
    A = _Args("sdpa_int4")
    b, hq, d = _query_arg(A, q, cache)
    if workspace is None:
        workspace = partials_buffers(b, hq, d, skv, chunk, device=q.device)
    m, l, acc = _workspace_arg(A, workspace, b, hq, d, num_chunks(skv, chunk))
    out = _out_arg(A, out, b, hq, d, q.device)
    A.devices(cache.device)
    cs = cache.c_struct()
    _check("kvq_sdpa_int4",
           lib().kvq_sdpa_int4(C.byref(cs), int(skv), _ptr(q), _dtype_code(q), hq, float(softmax_scale),
                               int(chunk), _ptr(m), _ptr(l), _ptr(acc), _ptr(out), int(kernel), _stream(stream)))
    return out


def _step_args(fn, cache, length, k_new, v_new, q, chunk, out, workspace):
    A = _Args(fn)
    _rows_arg(A, "k_new", k_new, cache, allow_3d=True)
    _rows_arg(A, "v_new", v_new, cache, allow_3d=True)
    if v_new.dtype != k_new.dtype:
        _fail(fn, "k_new and v_new must have the same dtype")
    b, hq, d = _query_arg(A, q, cache)
    if workspace is None:
        workspace = partials_buffers(b, hq, d, length + 1, chunk, device=q.device)
    ws = _workspace_arg(A, workspace, b, hq, d, num_chunks(length + 1, chunk))
    out = _out_arg(A, out, b, hq, d, q.device)
    A.devices(cache.device)
    return hq, ws, out


def decode_step(cache: QuantKVCache, length: int, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                softmax_scale: float, chunk: int = 512, out: torch.Tensor | None = None, workspace=None,
                kernel: int = KERNEL_AUTO, stream=None, events=None):
    """kvq_decode_step: append k_new, v_new ([B][Hkv][D] or [B][Hkv][1][D]) at
    row `length`, then attention over length + 1 rows; returns out [B][Hq][D].
    events: optional (start, stop) torch.cuda.Event recorded in the attention
    kernel's own dispatch (kvq_decode_step_timed)."""
    hq, (m, l, acc), out = _step_args("decode_step", cache, length, k_new, v_new, q, chunk, out, workspace)
    cs = cache.c_struct()
    args = (C.byref(cs), int(length), _ptr(k_new), _ptr(v_new), _dtype_code(k_new), _ptr(q), _dtype_code(q), hq,
            float(softmax_scale), int(chunk), _ptr(m), _ptr(l), _ptr(acc), _ptr(out), int(kernel), _stream(stream))
    if events is None:
        _check("kvq_decode_step", lib().kvq_decode_step(*args))
    else:
        _check("kvq_decode_step_timed",
               lib().kvq_decode_step_timed(*args, _event_handle(events[0]), _event_handle(events[1])))
    return out


def sdpa_int4_prefill(cache: QuantKVCache, q_start: int, q: torch.Tensor, softmax_scale: float,
                      out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """kvq_sdpa_int4_prefill: q [B][Hq][Sq][D] fp16 or fp32 contiguous, the queries of
    positions q_start .. q_start + Sq - 1 (their K/V rows already appended);
    returns out [B][Hq][Sq][D] fp32."""
    A = _Args("sdpa_int4_prefill")
    _query_arg(A, q, cache, dims=4)
    b, hq, sq, d = q.shape
    if out is None:
        out = torch.empty((b, hq, sq, d), dtype=torch.float32, device=q.device)
    A.need("out", out, (b, hq, sq, d), _F32)
    A.devices(cache.device)
    cs = cache.c_struct()
    _check("kvq_sdpa_int4_prefill",
           lib().kvq_sdpa_int4_prefill(C.byref(cs), int(q_start), int(sq), _ptr(q), _dtype_code(q), hq,
                                       float(softmax_scale), _ptr(out), _stream(stream)))
    return out


def decode_step_rotated(cache: QuantKVCache, length: int, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                        softmax_scale: float, chunk: int = 512, out: torch.Tensor | None = None, workspace=None,
                        kernel: int = KERNEL_AUTO, stream=None):
    """kvq_decode_step_rotated: the decode step on a Hadamard-rotated cache
    (fp16 k_new, v_new; q and out in the original coordinates); returns out
    [B][Hq][D] fp32."""
    hq, (m, l, acc), out = _step_args("decode_step_rotated", cache, length, k_new, v_new, q, chunk, out, workspace)
    cs = cache.c_struct()
    _check("kvq_decode_step_rotated",
           lib().kvq_decode_step_rotated(C.byref(cs), int(length), _ptr(k_new), _ptr(v_new), _dtype_code(k_new),
                                         _ptr(q), _dtype_code(q), hq, float(softmax_scale), int(chunk), _ptr(m),
                                         _ptr(l), _ptr(acc), _ptr(out), int(kernel), _stream(stream)))
    return out


def decode_workspace_bytes(cache: QuantKVCache, hq: int, max_rows: int) -> int:
    """kvq_decode_workspace_bytes: workspace bytes of decode_step_single_launch
    for steps over at most max_rows rows."""
    cs = cache.c_struct()
    n = int(lib().kvq_decode_workspace_bytes(C.byref(cs), int(hq), int(max_rows)))
    if n <= 0:
        _fail("decode_workspace_bytes", "invalid cache or sizes (Hq %d, max_rows %d)" % (hq, max_rows))
    return n


def decode_workspace(cache: QuantKVCache, hq: int, max_rows: int) -> torch.Tensor:
    """A zeroed workspace (uint8 device tensor) for decode_step_single_launch
    over at most max_rows rows; every call leaves its counters zero again."""
    n = decode_workspace_bytes(cache, hq, max_rows)
    return torch.zeros((n + 15) // 16 * 16, dtype=torch.uint8, device=cache.device)


def decode_step_single_launch(cache: QuantKVCache, length: int, k_new: torch.Tensor, v_new: torch.Tensor,
                              q: torch.Tensor, softmax_scale: float, workspace: torch.Tensor | None = None,
                              out: torch.Tensor | None = None, stream=None, events=None):
    """kvq_decode_step_single_launch: append k_new, v_new ([B][Hkv][D] or
    [B][Hkv][1][D]) at row `length`, then attention over length + 1 rows with
    the split-K merge inside the same launch; returns out [B][Hq][D] fp32.
    workspace: a uint8 device tensor from decode_workspace() (zeroed once,
    reused across calls on one stream). events: optional (start, stop)
    torch.cuda.Event recorded in the kernel's own dispatch."""
    fn = "decode_step_single_launch"
    A = _Args(fn)
    _rows_arg(A, "k_new", k_new, cache, allow_3d=True)
    _rows_arg(A, "v_new", v_new, cache, allow_3d=True)
    if v_new.dtype != k_new.dtype:
        _fail(fn, "k_new and v_new must have the same dtype")
    b, hq, d = _query_arg(A, q, cache)
    if workspace is None:
        workspace = decode_workspace(cache, hq, length + 1)
    need = decode_workspace_bytes(cache, hq, length + 1)
    A.need("workspace", workspace, None, (torch.uint8,), need)
    out = _out_arg(A, out, b, hq, d, q.device)
    A.devices(cache.device)
    ev = (None, None) if events is None else (_event_handle(events[0]), _event_handle(events[1]))
    cs = cache.c_struct()
    _check("kvq_decode_step_single_launch",
           lib().kvq_decode_step_single_launch(C.byref(cs), int(length), _ptr(k_new), _ptr(v_new), _dtype_code(k_new),
                                               _ptr(q), _dtype_code(q), hq, float(softmax_scale), _ptr(workspace),
                                               int(workspace.numel()), _ptr(out), _stream(stream), ev[0], ev[1]))
    return out


def decode_step_noalloc(cache: QuantKVCache, length: int, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                        softmax_scale: float, chunk: int = 512, out: torch.Tensor | None = None,
                        kernel: int = KERNEL_AUTO, stream=None):
    """kvq_decode_step_noalloc: kvq_decode_step with its partials in the
    library's static device scratch (no workspace; the library allocates
    nothing). Pass `out` to allocate nothing here either; returns out
    [B][Hq][D] fp32."""
    fn = "decode_step_noalloc"
    A = _Args(fn)
    _rows_arg(A, "k_new", k_new, cache, allow_3d=True)
    _rows_arg(A, "v_new", v_new, cache, allow_3d=True)
    if v_new.dtype != k_new.dtype:
        _fail(fn, "k_new and v_new must have the same dtype")
    b, hq, d = _query_arg(A, q, cache)
    out = _out_arg(A, out, b, hq, d, q.device)
    A.devices(cache.device)
    cs = cache.c_struct()
    _check("kvq_decode_step_noalloc",
           lib().kvq_decode_step_noalloc(C.byref(cs), int(length), _ptr(k_new), _ptr(v_new), _dtype_code(k_new),
                                         _ptr(q), _dtype_code(q), hq, float(softmax_scale), int(chunk), _ptr(out),
                                         int(kernel), _stream(stream)))
    return out
