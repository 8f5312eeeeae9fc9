"""ctypes binding of libwf_chunk_attn.so (argument marshalling only).

Every computation happens in the HIP library; this module only turns torch
tensors into device pointers and streams, and status codes into exceptions.
If the library has not been built the import of the first entry point fails
loudly -- there is no fallback implementation.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwf_chunk_attn.so")

WF_OK, WF_ERR_INVALID_ARG, WF_ERR_UNSUPPORTED, WF_ERR_CAPACITY, WF_ERR_RANGE, WF_ERR_HIP = range(6)
WF_F32, WF_BF16, WF_FP8_E4M3 = 0, 1, 2
WF_MAX_TABLE_LEN = 256
WF_MAX_CHUNKS = 64
WF_SCALE_BLOCK = 128
WF_EVICT_POISON = 1

STATUS_NAMES = {0: "WF_OK", 1: "WF_ERR_INVALID_ARG", 2: "WF_ERR_UNSUPPORTED", 3: "WF_ERR_CAPACITY",
                4: "WF_ERR_RANGE", 5: "WF_ERR_HIP"}
DTYPE_CODES = {"f32": WF_F32, "bf16": WF_BF16, "fp8": WF_FP8_E4M3}
TORCH_STORAGE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}


class WfError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), message))
        self.status = status


class wf_kv_cache(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("page_table", ctypes.POINTER(ctypes.c_int32)),
        ("table_len", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("start", ctypes.c_int64),
        ("end", ctypes.c_int64),
    ]


class wf_attn_plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("kernel", "schedule", "grid", "items", "rows_per_item", "parts",
                                               "tail_tiles", "tails_per_block")]


KERNEL_NAMES = {0: "f32", 1: "staged_bf16", 2: "staged_fp8", 3: "dma_bf16", 4: "dma_fp8"}
SCHEDULE_NAMES = {0: "per_tile", 1: "split"}

_lib = None


def lib():
    """Load the built library (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libwf_chunk_attn.so is not built; run `python -m chunk_causal_dit_wf_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(wf_kv_cache)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        L.wf_kv_cache_check.argtypes = [P]
        L.wf_kv_cache_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_uint64)]
        L.wf_kv_append.argtypes = [P, i64, i32, vp, vp, vp, vp, vp]
        L.wf_kv_evict.argtypes = [P, i32, ctypes.c_uint32, vp]
        L.wf_kv_append_quantize.argtypes = [P, i64, i32, vp, vp, vp]
        L.wf_chunk_attn_fwd.argtypes = [P, vp, i32, vp, vp, i32, ctypes.POINTER(i32), ctypes.POINTER(i64),
                                        ctypes.POINTER(i64), f32, vp, ctypes.c_uint64, vp]
        L.wf_chunk_attn_workspace_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_uint64)]
        L.wf_chunk_attn_fwd_noalloc.argtypes = [P, vp, i32, vp, vp, i32, ctypes.POINTER(i32), ctypes.POINTER(i64),
                                                ctypes.POINTER(i64), f32, vp]
        L.wf_chunk_attn_plan.argtypes = [P, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i64), ctypes.POINTER(i64),
                                         ctypes.c_uint64, ctypes.POINTER(wf_attn_plan)]
        L.wf_stream_copy.argtypes = [vp, vp, ctypes.c_uint64, vp]
        for name in ("wf_kv_cache_check", "wf_kv_cache_bytes", "wf_kv_append", "wf_kv_evict", "wf_chunk_attn_fwd",
                     "wf_chunk_attn_workspace_bytes", "wf_kv_append_quantize", "wf_chunk_attn_plan", "wf_chunk_attn_fwd_noalloc",
                     "wf_stream_copy"):
            getattr(L, name).restype = ctypes.c_int
        L.wf_last_error.restype = ctypes.c_char_p
        L.wf_last_error.argtypes = []
        L.wf_version.restype = ctypes.c_char_p
        L.wf_version.argtypes = []
        _lib = L
    return _lib


def _check(status):
    if status != WF_OK:
        raise WfError(status, lib().wf_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    if torch.cuda.is_available():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(None)


class KVCache:
    """One layer's paged ring KV cache: torch-owned device buffers + the C descriptor.

    Buffers follow the layout declared in include/wf_chunk_attn.h:
      k [num_pages, H, page_size, D], v [num_pages, H, D, page_size],
      k_scale / v_scale [num_pages, H, ceil(page_size/128)] float32 (E4M3FN only).
    """

    def __init__(self, num_pages, page_size, num_heads, head_dim, dtype, page_table, device="cuda",
                 k=None, v=None, k_scale=None, v_scale=None):
        self.dtype = dtype
        st = TORCH_STORAGE[dtype]
        self.table = (ctypes.c_int32 * len(page_table))(*[int(x) for x in page_table])
        nblk = -(-page_size // WF_SCALE_BLOCK)
        self.k = k if k is not None else torch.zeros((num_pages, num_heads, page_size, head_dim), dtype=st, device=device)
        self.v = v if v is not None else torch.zeros((num_pages, num_heads, head_dim, page_size), dtype=st, device=device)
        if dtype == "fp8":
            self.k_scale = k_scale if k_scale is not None else torch.ones((num_pages, num_heads, nblk), dtype=torch.float32, device=device)
            self.v_scale = v_scale if v_scale is not None else torch.ones((num_pages, num_heads, nblk), dtype=torch.float32, device=device)
        else:
            self.k_scale = self.v_scale = None
        self.c = wf_kv_cache(
            k=self.k.data_ptr(), v=self.v.data_ptr(),
            k_scale=None if self.k_scale is None else self.k_scale.data_ptr(),
            v_scale=None if self.v_scale is None else self.v_scale.data_ptr(),
            page_table=ctypes.cast(self.table, ctypes.POINTER(ctypes.c_int32)),
            table_len=len(page_table), num_pages=num_pages, page_size=page_size, num_heads=num_heads,
            head_dim=head_dim, kv_dtype=DTYPE_CODES[dtype], start=0, end=0)

    @property
    def start(self):
        return self.c.start

    @property
    def end(self):
        return self.c.end

    @property
    def capacity(self):
        return self.c.table_len * self.c.page_size


def wf_kv_cache_check(cache):
    _check(lib().wf_kv_cache_check(ctypes.byref(cache.c)))


def wf_kv_cache_bytes(cache):
    kb, sb = ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib().wf_kv_cache_bytes(ctypes.byref(cache.c), ctypes.byref(kb), ctypes.byref(sb)))
    return kb.value, sb.value


def wf_kv_append(cache, pos, k_new, v_new, k_scale_new=None, v_scale_new=None, stream=None):
    """Write tokens [pos, pos + n) (k_new/v_new: [n, H, D] device tensors in the cache dtype)."""
    n = int(k_new.shape[0])
    _check(lib().wf_kv_append(ctypes.byref(cache.c), int(pos), n, _ptr(k_new), _ptr(v_new),
                              _ptr(k_scale_new), _ptr(v_scale_new), _stream(stream)))


def wf_kv_append_quantize(cache, pos, k_new, v_new, stream=None):
    """Quantise bf16 rows k_new/v_new [n, H, D] to E4M3FN (per page, head, 128-token block) and append."""
    n = int(k_new.shape[0])
    _check(lib().wf_kv_append_quantize(ctypes.byref(cache.c), int(pos), n, _ptr(k_new), _ptr(v_new),
                                       _stream(stream)))


def wf_kv_evict(cache, n, poison=False, stream=None):
    _check(lib().wf_kv_evict(ctypes.byref(cache.c), int(n), WF_EVICT_POISON if poison else 0, _stream(stream)))


def wf_stream_copy(src, dst, nbytes=None, stream=None):
    """Measurement aid: copy nbytes (default: all of src) from tensor src to tensor dst."""
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    _check(lib().wf_stream_copy(_ptr(src), _ptr(dst), n, _stream(stream)))


def wf_chunk_attn_workspace_bytes(cache):
    b = ctypes.c_uint64()
    _check(lib().wf_chunk_attn_workspace_bytes(ctypes.byref(cache.c), ctypes.byref(b)))
    return b.value


_workspaces = {}


def workspace_for(cache, device):
    """A cached device workspace large enough for the balanced schedule (None if the cache needs none).
    One buffer per device: calls that use it must be ordered on one stream."""
    n = wf_chunk_attn_workspace_bytes(cache)
    if n == 0:
        return None
    key = torch.device(device)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < n:
        ws = torch.empty(n, dtype=torch.uint8, device=key)
        _workspaces[key] = ws
    return ws


def wf_chunk_attn_fwd(cache, q, q_off, kv_begin, kv_end, softmax_scale=0.0, o=None, lse=None,
                      return_lse=False, workspace="auto", stream=None):
    """Chunk-wise causal attention.  q: [Nq, H, D] device tensor (f32 or bf16).

    workspace: "auto" (a cached per-device buffer: balanced schedule where the cache dtype uses one),
    None (one workgroup per query tile) or a uint8 device tensor.
    Returns o (and lse [H, Nq] float32 when return_lse or lse is given).
    """
    nc = len(kv_begin)
    qo = (ctypes.c_int32 * (nc + 1))(*[int(x) for x in q_off])
    kb = (ctypes.c_int64 * nc)(*[int(x) for x in kv_begin])
    ke = (ctypes.c_int64 * nc)(*[int(x) for x in kv_end])
    qd = _q_dtype(q)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    if isinstance(workspace, str):
        workspace = workspace_for(cache, q.device) if q.is_cuda else None
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().wf_chunk_attn_fwd(ctypes.byref(cache.c), _ptr(q), qd, _ptr(o), _ptr(lse), nc, qo, kb, ke,
                                   float(softmax_scale), _ptr(workspace), wsb, _stream(stream)))
    return (o, lse) if lse is not None else o


def wf_chunk_attn_fwd_noalloc(cache, q, q_off, kv_begin, kv_end, o, lse=None, softmax_scale=0.0, stream=None):
    """wf_chunk_attn_fwd without a workspace and without any allocation: the caller passes o (and lse)."""
    nc = len(kv_begin)
    qo = (ctypes.c_int32 * (nc + 1))(*[int(x) for x in q_off])
    kb = (ctypes.c_int64 * nc)(*[int(x) for x in kv_begin])
    ke = (ctypes.c_int64 * nc)(*[int(x) for x in kv_end])
    _check(lib().wf_chunk_attn_fwd_noalloc(ctypes.byref(cache.c), _ptr(q), _q_dtype(q), _ptr(o), _ptr(lse), nc, qo,
                                           kb, ke, float(softmax_scale), _stream(stream)))
    return o


def _q_dtype(q):
    if q.dtype == torch.float32:
        return WF_F32
    if q.dtype == torch.bfloat16:
        return WF_BF16
    raise WfError(WF_ERR_UNSUPPORTED, "q dtype %s" % q.dtype)


def wf_chunk_attn_plan(cache, q_off, kv_begin, kv_end, q_dtype="bf16", workspace_bytes=0):
    """The launch wf_chunk_attn_fwd would make (kernel, schedule, grid, ...), as a dict."""
    nc = len(kv_begin)
    qo = (ctypes.c_int32 * (nc + 1))(*[int(x) for x in q_off])
    kb = (ctypes.c_int64 * nc)(*[int(x) for x in kv_begin])
    ke = (ctypes.c_int64 * nc)(*[int(x) for x in kv_end])
    out = wf_attn_plan()
    _check(lib().wf_chunk_attn_plan(ctypes.byref(cache.c), DTYPE_CODES[q_dtype], nc, qo, kb, ke,
                                    int(workspace_bytes), ctypes.byref(out)))
    d = {n: getattr(out, n) for n, _ in wf_attn_plan._fields_}
    d["kernel"] = KERNEL_NAMES[d["kernel"]]
    d["schedule"] = SCHEDULE_NAMES[d["schedule"]]
    return d


def version():
    return lib().wf_version().decode()
