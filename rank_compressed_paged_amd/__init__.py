"""Python binding of libstarkv (STAR-KV decode over a low-rank paged KV cache).

Argument marshalling only: every step of the path runs in the HIP library
(include/starkv.h).  Tensors are torch tensors on the GPU; torch provides
device memory and the current stream, nothing else.  If the compiled library
is missing, every call raises - there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "Dims", "StarkvError", "load_library", "library_path", "status_string",
    "decode_workspace_size", "decode", "decode_noalloc", "decode_step", "uncompressed_decode", "append", "prefill_workspace_size", "prefill", "profile_begin",
    "profile_end", "stream_read_probe", "check_block_tables",
    "BLOCK_SIZE",
]

BLOCK_SIZE = 16
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libstarkv.so"

STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "HIP"}


class StarkvError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {status_string(code)}")


class Dims(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("rank_k", ctypes.c_int32),
        ("rank_v", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
    ]

    @classmethod
    def make(cls, heads, head_dim, rank_k, rank_v, num_blocks, max_blocks_per_seq, block_size=BLOCK_SIZE,
             kv_heads=None):
        return cls(heads, head_dim, rank_k, rank_v, block_size, num_blocks, max_blocks_per_seq,
                   heads if kv_heads is None else kv_heads)


_lib = None


def library_path() -> str:
    return os.environ.get("STARKV_LIBRARY", os.path.join(_HERE, _LIB_NAME))


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libstarkv.so (built by rank_compressed_paged_amd.build)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path()
    if not os.path.exists(p):
        raise RuntimeError(f"libstarkv not built: {p} is missing (run python -m rank_compressed_paged_amd.build)")
    lib = ctypes.CDLL(p)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    dp = ctypes.POINTER(Dims)
    lib.starkv_status_string.argtypes = [ctypes.c_int]
    lib.starkv_status_string.restype = ctypes.c_char_p
    lib.starkv_decode_workspace_size.argtypes = [dp, i32, i32]
    lib.starkv_decode_workspace_size.restype = sz
    lib.starkv_decode.argtypes = [dp, i32, i32, vp, vp, vp, vp, vp, vp, vp, f32, vp, sz, vp, vp]
    lib.starkv_decode.restype = ctypes.c_int
    lib.starkv_decode_noalloc.argtypes = [dp, i32, i32, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp]
    lib.starkv_decode_noalloc.restype = ctypes.c_int
    lib.starkv_decode_step.argtypes = [dp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp,
                                       sz, vp, vp]
    lib.starkv_decode_step.restype = ctypes.c_int
    lib.starkv_uncompressed_decode_workspace_size.argtypes = [dp, i32, i32]
    lib.starkv_uncompressed_decode_workspace_size.restype = sz
    lib.starkv_uncompressed_decode.argtypes = [dp, i32, i32, vp, vp, vp, vp, vp, f32, vp, sz, vp, vp]
    lib.starkv_uncompressed_decode.restype = ctypes.c_int
    lib.starkv_prefill_workspace_size.argtypes = [dp, i32, i32, i32]
    lib.starkv_prefill_workspace_size.restype = sz
    lib.starkv_prefill.argtypes = [dp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, sz, vp, vp]
    lib.starkv_prefill.restype = ctypes.c_int
    lib.starkv_append.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.starkv_append.restype = ctypes.c_int
    lib.starkv_profile_begin.argtypes = []
    lib.starkv_profile_begin.restype = ctypes.c_int
    lib.starkv_profile_end.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)]
    lib.starkv_profile_end.restype = ctypes.c_int
    lib.starkv_stream_read_probe.argtypes = [vp, sz, vp, i32, i32, vp]
    lib.starkv_stream_read_probe.restype = ctypes.c_int
    lib.starkv_check_block_tables.argtypes = [dp, i32, vp, vp, vp, vp]
    lib.starkv_check_block_tables.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def status_string(code: int) -> str:
    try:
        return load_library().starkv_status_string(int(code)).decode()
    except RuntimeError:
        return STATUS.get(int(code), f"status {code}")


def _check(code: int, what: str):
    if code != 0:
        raise StarkvError(code, what)


def _need(t, name, dtype, ndim=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _torch_stream(stream, device):
    """The torch Stream object of `stream` (None = the current stream)."""
    import torch
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _scratch(nbytes, device, stream):
    """Workspace for one call on `stream`.  It is allocated from the caching
    allocator's pool of that stream, so once the call returns and the tensor
    is dropped the memory is reused only by work ordered after the call's
    kernels on the same stream."""
    import torch
    s = _torch_stream(stream, device)
    with torch.cuda.stream(s):
        return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _own_out(out, device, stream):
    """A tensor the library writes on a stream other than the current one must
    not be recycled by the allocator before that stream gets there."""
    import torch
    s = _torch_stream(stream, device)
    if s != torch.cuda.current_stream(device):
        out.record_stream(s)


def dims_of(k_cache, v_cache, block_tables, head_dim, heads=None):
    """Dims from the cache shapes; `heads` = query heads (default: the cache's key/value heads)."""
    nb, kv_heads, bs, rank_k = k_cache.shape
    rank_v = v_cache.shape[1]
    return Dims.make(kv_heads if heads is None else heads, head_dim, rank_k, rank_v, nb, block_tables.shape[1],
                     block_size=bs, kv_heads=kv_heads)


def decode_workspace_size(dims: Dims, batch: int, max_context_len: int) -> int:
    return int(load_library().starkv_decode_workspace_size(ctypes.byref(dims), batch, max_context_len))


def decode(q, b_k, b_v, k_cache, v_cache, block_tables, context_lens, scale, *,
           max_context_len=None, workspace=None, out=None, stream=None):
    """out[b, h, :] of single-query attention over the latent paged cache.

    q [B, H, d] fp16; b_k [H_kv, r_k, d] fp16; b_v [r_v, H_kv*d] fp16;
    k_cache [NB, H_kv, 16, r_k] fp16; v_cache [NB, r_v, 16] fp16 (H_kv = H,
    or a divisor of H for grouped query heads);
    block_tables [B, MB] int32; context_lens [B] int32.  max_context_len
    defaults to 16*MB (no host sync).  Returns out [B, H, d] fp16.
    """
    import torch
    lib = load_library()
    batch, heads, d = q.shape
    dims = dims_of(k_cache, v_cache, block_tables, d, heads=heads)
    kvh = dims.num_kv_heads
    if max_context_len is None:
        max_context_len = BLOCK_SIZE * block_tables.shape[1]
    ptrs = [
        _need(q, "q", torch.float16, 3), _need(b_k, "b_k", torch.float16, 3),
        _need(b_v, "b_v", torch.float16, 2), _need(k_cache, "k_cache", torch.float16, 4),
        _need(v_cache, "v_cache", torch.float16, 3), _need(block_tables, "block_tables", torch.int32, 2),
        _need(context_lens, "context_lens", torch.int32, 1),
    ]
    if block_tables.shape[0] != batch or context_lens.shape[0] != batch:
        raise ValueError("block_tables / context_lens rows must match q's batch")
    if kvh < 1 or heads % kvh != 0:
        raise ValueError("query heads must be a multiple of the cache's key/value heads")
    if tuple(b_k.shape) != (kvh, dims.rank_k, d) or tuple(b_v.shape) != (dims.rank_v, kvh * d):
        raise ValueError("projection shapes do not match the caches")
    if tuple(v_cache.shape) != (dims.num_blocks, dims.rank_v, BLOCK_SIZE) or k_cache.shape[2] != BLOCK_SIZE:
        raise ValueError("cache shapes do not match the paged layout")
    need = lib.starkv_decode_workspace_size(ctypes.byref(dims), batch, int(max_context_len))
    if need == 0:
        _check(1, "starkv_decode_workspace_size")
    if workspace is None:
        workspace = _scratch(need + 256, q.device, stream)
    ws_ptr = _need(workspace, "workspace", torch.uint8, 1)
    pad = (-ws_ptr) % 256
    if out is None:
        out = torch.empty_like(q)
        _own_out(out, q.device, stream)
    optr = _need(out, "out", torch.float16, 3)
    code = lib.starkv_decode(ctypes.byref(dims), batch, int(max_context_len), *ptrs[:5], ptrs[5], ptrs[6],
                             float(scale), ctypes.c_void_p(ws_ptr + pad), workspace.numel() - pad,
                             ctypes.c_void_p(optr), _stream(stream))
    _check(code, "starkv_decode")
    return out


def decode_step(k_new, v_new, w_k, w_v, token_seq, token_pos, q, b_k, b_v, k_cache, v_cache, block_tables,
                context_lens, scale, *, max_context_len=None, workspace=None, out=None, stream=None):
    """append(k_new, v_new, w_k, w_v, ..., token_seq, token_pos) then decode(...),
    in one library call whose first launch holds the append and the query
    projection (starkv_decode_step).  context_lens count the new tokens.
    Arguments as in append() and decode(); returns out [B, H, d] fp16."""
    import torch
    lib = load_library()
    batch, heads, d = q.shape
    n = k_new.shape[0]
    dims = dims_of(k_cache, v_cache, block_tables, d, heads=heads)
    kvh = dims.num_kv_heads
    if max_context_len is None:
        max_context_len = BLOCK_SIZE * block_tables.shape[1]
    ptrs = [
        _need(k_new, "k_new", torch.float16, 3), _need(v_new, "v_new", torch.float16, 3),
        _need(w_k, "w_k", torch.float16, 3), _need(w_v, "w_v", torch.float16, 2),
        _need(token_seq, "token_seq", torch.int32, 1), _need(token_pos, "token_pos", torch.int32, 1),
        _need(q, "q", torch.float16, 3), _need(b_k, "b_k", torch.float16, 3), _need(b_v, "b_v", torch.float16, 2),
        _need(k_cache, "k_cache", torch.float16, 4), _need(v_cache, "v_cache", torch.float16, 3),
        _need(block_tables, "block_tables", torch.int32, 2), _need(context_lens, "context_lens", torch.int32, 1),
    ]
    if tuple(k_new.shape) != (n, kvh, d) or tuple(v_new.shape) != (n, kvh, d):
        raise ValueError("new rows must be [n, H_kv, d]")
    if token_seq.shape[0] != n or token_pos.shape[0] != n:
        raise ValueError("token_seq / token_pos must have one entry per new row")
    if block_tables.shape[0] != batch or context_lens.shape[0] != batch:
        raise ValueError("block_tables / context_lens rows must match q's batch")
    if tuple(w_k.shape) != (kvh, dims.rank_k, d) or tuple(w_v.shape) != (dims.rank_v, kvh * d):
        raise ValueError("down-projection shapes do not match the caches")
    if tuple(b_k.shape) != (kvh, dims.rank_k, d) or tuple(b_v.shape) != (dims.rank_v, kvh * d):
        raise ValueError("projection shapes do not match the caches")
    need = lib.starkv_decode_workspace_size(ctypes.byref(dims), batch, int(max_context_len))
    if need == 0:
        _check(1, "starkv_decode_workspace_size")
    if workspace is None:
        workspace = _scratch(need + 256, q.device, stream)
    ws_ptr = _need(workspace, "workspace", torch.uint8, 1)
    pad = (-ws_ptr) % 256
    if out is None:
        out = torch.empty_like(q)
        _own_out(out, q.device, stream)
    optr = _need(out, "out", torch.float16, 3)
    code = lib.starkv_decode_step(ctypes.byref(dims), batch, int(max_context_len), n,
                                  *[ctypes.c_void_p(p) for p in ptrs], float(scale), ctypes.c_void_p(ws_ptr + pad),
                                  workspace.numel() - pad, ctypes.c_void_p(optr), _stream(stream))
    _check(code, "starkv_decode_step")
    return out


def decode_noalloc(q, b_k, b_v, k_cache, v_cache, block_tables, context_lens, scale, out, *,
                   max_context_len=None, stream=None):
    """decode() through starkv_decode_noalloc: no workspace, the library's own
    fixed per-GPU scratch instead (calls on one GPU must not overlap).  `out`
    [B, H, d] fp16 is required, so nothing is allocated here either."""
    import torch
    lib = load_library()
    batch, heads, d = q.shape
    dims = dims_of(k_cache, v_cache, block_tables, d, heads=heads)
    if max_context_len is None:
        max_context_len = BLOCK_SIZE * block_tables.shape[1]
    ptrs = [
        _need(q, "q", torch.float16, 3), _need(b_k, "b_k", torch.float16, 3),
        _need(b_v, "b_v", torch.float16, 2), _need(k_cache, "k_cache", torch.float16, 4),
        _need(v_cache, "v_cache", torch.float16, 3), _need(block_tables, "block_tables", torch.int32, 2),
        _need(context_lens, "context_lens", torch.int32, 1),
    ]
    if block_tables.shape[0] != batch or context_lens.shape[0] != batch:
        raise ValueError("block_tables / context_lens rows must match q's batch")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    optr = _need(out, "out", torch.float16, 3)
    code = lib.starkv_decode_noalloc(ctypes.byref(dims), batch, int(max_context_len),
                                     *[ctypes.c_void_p(p) for p in ptrs], float(scale), ctypes.c_void_p(optr),
                                     _stream(stream))
    _check(code, "starkv_decode_noalloc")
    return out


def uncompressed_decode(q, k_cache, v_cache, block_tables, context_lens, scale, *,
                        max_context_len=None, workspace=None, out=None, stream=None):
    """The baseline the latent path is compared with: single-query attention
    over a plain paged fp16 cache of full-width keys and values.

    q [B, H, d] fp16; k_cache, v_cache [NB, H_kv, 16, d] fp16; block_tables
    [B, MB] int32; context_lens [B] int32.  Returns out [B, H, d] fp16.
    """
    import torch
    lib = load_library()
    batch, heads, d = q.shape
    nb, kvh, bs, d2 = k_cache.shape
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache / v_cache must be [NB, H_kv, 16, d] with q's head_dim")
    dims = Dims.make(heads, d, 1, 32, nb, block_tables.shape[1], block_size=bs, kv_heads=kvh)
    if max_context_len is None:
        max_context_len = BLOCK_SIZE * block_tables.shape[1]
    ptrs = [
        _need(q, "q", torch.float16, 3), _need(k_cache, "k_cache", torch.float16, 4),
        _need(v_cache, "v_cache", torch.float16, 4), _need(block_tables, "block_tables", torch.int32, 2),
        _need(context_lens, "context_lens", torch.int32, 1),
    ]
    if block_tables.shape[0] != batch or context_lens.shape[0] != batch:
        raise ValueError("block_tables / context_lens rows must match q's batch")
    need = lib.starkv_uncompressed_decode_workspace_size(ctypes.byref(dims), batch, int(max_context_len))
    if need == 0:
        _check(2 if heads % kvh == 0 else 1, "starkv_uncompressed_decode_workspace_size")
    if workspace is None:
        workspace = _scratch(need + 256, q.device, stream)
    ws_ptr = _need(workspace, "workspace", torch.uint8, 1)
    pad = (-ws_ptr) % 256
    if out is None:
        out = torch.empty_like(q)
        _own_out(out, q.device, stream)
    optr = _need(out, "out", torch.float16, 3)
    code = lib.starkv_uncompressed_decode(ctypes.byref(dims), batch, int(max_context_len),
                                          *[ctypes.c_void_p(p) for p in ptrs], float(scale),
                                          ctypes.c_void_p(ws_ptr + pad), workspace.numel() - pad,
                                          ctypes.c_void_p(optr), _stream(stream))
    _check(code, "starkv_uncompressed_decode")
    return out


def prefill_workspace_size(dims: Dims, batch: int, num_queries: int, max_context_len: int) -> int:
    return int(load_library().starkv_prefill_workspace_size(ctypes.byref(dims), batch, num_queries,
                                                              max_context_len))


def prefill(q, b_k, b_v, k_cache, v_cache, block_tables, query_start, context_lens, scale, *,
            max_context_len=None, workspace=None, out=None, stream=None):
    """Causal attention of each sequence's chunk of new tokens over the latent cache.

    q [N, H, d] fp16: rows query_start[b] .. query_start[b+1]-1 belong to
    sequence b and are its last n_b positions (their latents already appended);
    query_start [B+1] int32, context_lens [B] int32 (device).  Other arguments
    as in decode().  max_context_len defaults to 16*MB.  Returns out [N, H, d].
    """
    import torch
    lib = load_library()
    rows, heads, d = q.shape
    batch = block_tables.shape[0]
    dims = dims_of(k_cache, v_cache, block_tables, d, heads=heads)
    kvh = dims.num_kv_heads
    if max_context_len is None:
        max_context_len = BLOCK_SIZE * block_tables.shape[1]
    ptrs = [
        _need(q, "q", torch.float16, 3), _need(b_k, "b_k", torch.float16, 3),
        _need(b_v, "b_v", torch.float16, 2), _need(k_cache, "k_cache", torch.float16, 4),
        _need(v_cache, "v_cache", torch.float16, 3), _need(block_tables, "block_tables", torch.int32, 2),
        _need(query_start, "query_start", torch.int32, 1), _need(context_lens, "context_lens", torch.int32, 1),
    ]
    if query_start.shape[0] != batch + 1 or context_lens.shape[0] != batch:
        raise ValueError("query_start needs B+1 entries and context_lens B")
    if kvh < 1 or heads % kvh != 0:
        raise ValueError("query heads must be a multiple of the cache's key/value heads")
    if tuple(b_k.shape) != (kvh, dims.rank_k, d) or tuple(b_v.shape) != (dims.rank_v, kvh * d):
        raise ValueError("projection shapes do not match the caches")
    if out is None:
        out = torch.empty_like(q)
        _own_out(out, q.device, stream)
    if rows == 0:
        return out
    need = lib.starkv_prefill_workspace_size(ctypes.byref(dims), batch, rows, int(max_context_len))
    if need == 0:
        _check(1, "starkv_prefill_workspace_size")
    if workspace is None:
        workspace = _scratch(need + 256, q.device, stream)
    ws_ptr = _need(workspace, "workspace", torch.uint8, 1)
    pad = (-ws_ptr) % 256
    optr = _need(out, "out", torch.float16, 3)
    code = lib.starkv_prefill(ctypes.byref(dims), batch, rows, int(max_context_len), *[ctypes.c_void_p(p) for p in ptrs],
                              float(scale), ctypes.c_void_p(ws_ptr + pad), workspace.numel() - pad,
                              ctypes.c_void_p(optr), _stream(stream))
    _check(code, "starkv_prefill")
    return out


def append(k, v, w_k, w_v, block_tables, token_seq, token_pos, k_cache, v_cache, *, stream=None):
    """Project new rows into latents and scatter them into the paged caches (in place).

    k, v [n, H_kv, d] fp16; w_k [H_kv, r_k, d] fp16; w_v [r_v, H_kv*d] fp16
    (output-major down-projections); token_seq / token_pos [n] int32.
    """
    import torch
    lib = load_library()
    n, heads, d = k.shape
    dims = dims_of(k_cache, v_cache, block_tables, d)
    if heads != dims.num_kv_heads:
        raise ValueError("k rows must have the cache's key/value heads")
    ptrs = [
        _need(k, "k", torch.float16, 3), _need(v, "v", torch.float16, 3),
        _need(w_k, "w_k", torch.float16, 3), _need(w_v, "w_v", torch.float16, 2),
        _need(block_tables, "block_tables", torch.int32, 2),
        _need(token_seq, "token_seq", torch.int32, 1), _need(token_pos, "token_pos", torch.int32, 1),
        _need(k_cache, "k_cache", torch.float16, 4), _need(v_cache, "v_cache", torch.float16, 3),
    ]
    if tuple(v.shape) != (n, heads, d) or token_seq.shape[0] != n or token_pos.shape[0] != n:
        raise ValueError("k, v, token_seq and token_pos must agree on n")
    if tuple(w_k.shape) != (heads, dims.rank_k, d) or tuple(w_v.shape) != (dims.rank_v, heads * d):
        raise ValueError("down-projection shapes do not match the caches")
    code = lib.starkv_append(ctypes.byref(dims), n, *[ctypes.c_void_p(p) for p in ptrs], _stream(stream))
    _check(code, "starkv_append")


def check_block_tables(block_tables, context_lens, dims: Dims, *, out=None, stream=None):
    """Count block-table violations a decode over these tables would hit
    (lengths outside [0, 16*MB], read entries outside [0, num_blocks)).

    Returns a device int32 tensor [1] (read it after the stream gets there)."""
    import torch
    bt = _need(block_tables, "block_tables", torch.int32, 2)
    cl = _need(context_lens, "context_lens", torch.int32, 1)
    batch = block_tables.shape[0]
    if context_lens.shape[0] != batch or block_tables.shape[1] != dims.max_blocks_per_seq:
        raise ValueError("block_tables / context_lens do not match the dims")
    if out is None:
        out = torch.empty(1, dtype=torch.int32, device=block_tables.device)
    op = _need(out, "out", torch.int32, 1)
    _check(load_library().starkv_check_block_tables(ctypes.byref(dims), batch, ctypes.c_void_p(bt),
                                                     ctypes.c_void_p(cl), ctypes.c_void_p(op), _stream(stream)),
           "starkv_check_block_tables")
    return out


def stream_read_probe(buf, sink, grid: int, block: int, stream=None):
    """Launch the HBM stream-read probe over the whole of `buf` (uint8, GPU)."""
    import torch
    p = _need(buf, "buf", torch.uint8, 1)
    sp = _need(sink, "sink", torch.int32, 1)
    if sink.numel() < grid:
        raise ValueError("sink needs one int32 per workgroup")
    _check(load_library().starkv_stream_read_probe(ctypes.c_void_p(p), buf.numel() // 16 * 16, ctypes.c_void_p(sp),
                                                    grid, block, _stream(stream)), "starkv_stream_read_probe")


def profile_begin():
    _check(load_library().starkv_profile_begin(), "starkv_profile_begin")


def profile_end():
    """(summed attention-kernel milliseconds, bracketed launches) since profile_begin()."""
    ms = ctypes.c_double()
    n = ctypes.c_int32()
    _check(load_library().starkv_profile_end(ctypes.byref(ms), ctypes.byref(n)), "starkv_profile_end")
    return ms.value, n.value
