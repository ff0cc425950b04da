"""Python binding of ``libpagedkv.so`` (the C ABI in ``include/pagedkv.h``).

Argument marshalling only: every step of the decode path runs in the library's HIP kernels.
Tensors supply device memory, ``torch.cuda.current_stream()`` supplies the stream. The
functions keep the C names. A missing library raises ``ImportError`` on first use; there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # loaded first: the library then binds to the HIP runtime torch already loaded

__all__ = [
    "PagedKVError", "paged_attn_decode", "paged_attn_decode_append", "kv_cache_append",
    "cow_block_copy", "kv_swap_out", "kv_swap_in", "kv_swap_out_dma", "kv_swap_in_dma",
    "swap_staging", "paged_attn_decode_shared_prefix",
    "shared_prefix_workspace", "paged_attn_extend", "paged_attn_decode_noalloc",
    "DECODE_STATIC_SCRATCH", "extend_workspace", "pkv_decode_workspace_size", "decode_workspace",
    "pkv_decode_auto_workers", "BlockPool", "timing_enable", "timing_query",
    "stream_read_probe", "mfma_rate_probe", "set_validate", "library_path", "load_library", "PKV_F32", "PKV_F16",
    "PKV_BF16", "PrefixIndex",
]

PKV_F32, PKV_F16, PKV_BF16 = 0, 1, 2
_DT = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16}
_ERRNAMES = {
    -1: "PKV_ERR_INVALID_ARG", -2: "PKV_ERR_UNSUPPORTED", -3: "PKV_ERR_WORKSPACE_TOO_SMALL",
    -4: "PKV_ERR_LAUNCH", -5: "PKV_ERR_POOL_EXHAUSTED", -6: "PKV_ERR_REFCOUNT",
    -7: "PKV_ERR_VALIDATION",
}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpagedkv.so")
_lib = None


class PagedKVError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_ERRNAMES.get(code, code)}: {msg}")
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def _declare(L):
    c_int, c_void, c_size, c_float = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
    P = ctypes.POINTER
    i32p = P(ctypes.c_int32)
    sig = {
        "pkv_last_error": (ctypes.c_char_p, []),
        "pkv_version": (ctypes.c_char_p, []),
        "pkv_decode_workspace_size": (c_size, [c_int] * 5),
        "pkv_decode_auto_workers": (c_int, []),
        "paged_attn_decode": (c_int, [c_void, c_int, c_void, c_void, c_void, c_int, c_void, c_int,
                                      c_void, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                      c_float, c_int, c_void, c_size, c_void]),
        "paged_attn_decode_noalloc": (c_int, [c_void, c_int, c_void, c_void, c_void, c_int,
                                              c_void, c_int, c_void, c_int, c_int, c_int, c_int,
                                              c_int, c_int, c_int, c_float, c_int, c_void]),
        "paged_attn_decode_append": (c_int, [c_void, c_int, c_void, c_void, c_void, c_int, c_void,
                                             c_void, c_void, c_int, c_void, c_int, c_int, c_int,
                                             c_int, c_int, c_int, c_int, c_float, c_int, c_void,
                                             c_size, c_void]),
        "kv_cache_append": (c_int, [c_void, c_void, c_int, c_void, c_void, c_void, c_void, c_int,
                                    c_void, c_int, c_int, c_int, c_int, c_int, c_int, c_void]),
        "cow_block_copy": (c_int, [c_void, c_void, c_int, c_void, c_void, c_void, c_int, c_int,
                                   c_int, c_int, c_int, c_void]),
        "pkv_shared_prefix_workspace_size": (c_size, [c_int, c_int, c_int, c_int, c_int, c_int]),
        "paged_attn_decode_shared_prefix": (c_int, [c_void, c_int, c_void, c_void, c_void, c_int,
                                                    c_void, c_int, c_void, c_int, c_void, c_int,
                                                    c_int, c_int, c_int, c_int, c_int, c_int,
                                                    c_float, c_int, c_void, c_size, c_void]),
        "pkv_extend_workspace_size": (c_size, [c_int, c_int, c_int, c_int, c_int, c_int, c_int]),
        "paged_attn_extend": (c_int, [c_void, c_int, c_void, c_void, c_int, c_int, c_void, c_void,
                                      c_int, c_void, c_int, c_void, c_int, c_int, c_int, c_int,
                                      c_int, c_int, c_int, c_float, c_void, c_size, c_void]),
        "kv_swap_out": (c_int, [c_void, c_void, c_int, c_void, c_void, c_int, c_void, c_void,
                                c_int, c_int, c_int, c_int, c_int, c_void]),
        "kv_swap_in": (c_int, [c_void, c_void, c_int, c_void, c_void, c_int, c_void, c_void,
                               c_int, c_int, c_int, c_int, c_int, c_void]),
        "pkv_swap_staging_size": (c_size, [c_int, c_int, c_int, c_int, c_int]),
        "kv_swap_out_dma": (c_int, [c_void, c_void, c_int, c_void, c_void, c_int, c_void, c_int,
                                    c_int, c_int, c_int, c_int, c_int, c_void, c_size, c_void]),
        "kv_swap_in_dma": (c_int, [c_void, c_void, c_int, c_void, c_void, c_int, c_int, c_void,
                                   c_int, c_int, c_int, c_int, c_int, c_void, c_size, c_void]),
        "pkv_prefix_index_create": (c_void, [c_void, c_int]),
        "pkv_prefix_index_destroy": (None, [c_void]),
        "pkv_prefix_index_match": (c_int, [c_void, i32p, c_int, i32p, c_int, P(c_int)]),
        "pkv_prefix_index_insert": (c_int, [c_void, i32p, c_int, i32p, P(c_int)]),
        "pkv_prefix_index_evict": (c_int, [c_void, c_int, i32p, P(c_int)]),
        "pkv_prefix_index_size": (c_int, [c_void]),
        "pkv_pool_create": (c_void, [c_int]),
        "pkv_pool_destroy": (None, [c_void]),
        "pkv_pool_alloc": (c_int, [c_void, i32p]),
        "pkv_pool_claim": (c_int, [c_void, ctypes.c_int32]),
        "pkv_pool_incref": (c_int, [c_void, ctypes.c_int32]),
        "pkv_pool_decref": (c_int, [c_void, ctypes.c_int32, P(c_int)]),
        "pkv_pool_refcount": (c_int, [c_void, ctypes.c_int32]),
        "pkv_pool_num_free": (c_int, [c_void]),
        "pkv_seq_prepare_write": (c_int, [c_void, i32p, c_int, c_int, c_int, i32p, i32p, i32p,
                                          i32p, i32p]),
        "pkv_seq_fork": (c_int, [c_void, i32p, i32p, c_int]),
        "pkv_seq_release": (c_int, [c_void, i32p, c_int]),
        "pkv_timing_enable": (c_int, [c_int]),
        "pkv_set_validate": (c_int, [c_int]),
        "pkv_timing_query": (c_int, [ctypes.c_char_p, P(ctypes.c_double), P(ctypes.c_int64)]),
        "pkv_stream_read_probe": (c_int, [c_void, c_size, c_void, c_void]),
        "pkv_mfma_rate_probe": (c_int, [c_int, c_int, c_void, c_void]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args


def load_library():
    """Load ``libpagedkv.so`` (once). Raises ImportError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with "
                              "`python -m paged_kv_cache_127_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        _declare(L)
        _lib = L
    return _lib


def _check(rc: int):
    if rc != 0:
        msg = load_library().pkv_last_error().decode(errors="replace")
        raise PagedKVError(rc, msg)
    return rc


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _kv_dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported cache dtype {t.dtype}")
    return _DT[t.dtype]


def pkv_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                              num_workers=0) -> int:
    return int(load_library().pkv_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads,
                                                         head_dim, num_workers))


def decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, num_workers=0,
                     device="cuda") -> torch.Tensor:
    """Allocate a decode workspace for these sizes."""
    n = pkv_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, num_workers)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def pkv_decode_auto_workers() -> int:
    return int(load_library().pkv_decode_auto_workers())


def paged_attn_decode(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor,
                      v_pool: torch.Tensor, block_tables: torch.Tensor,
                      context_lens: torch.Tensor, max_context_len: int, scale: float = 0.0,
                      num_workers: int = 0, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """out[s][h] = softmax(q[s][h] . K_s^T * scale) . V_s over the paged cache (C:
    ``paged_attn_decode``). Shapes: q, out [S][H_q][d]; k_pool, v_pool [N][H_kv][B][d];
    block_tables int32 [S][max_blocks]; context_lens int32 [S]."""
    L = load_library()
    kdt = _kv_dtype(k_pool)
    if q.dim() != 3 or k_pool.dim() != 4 or v_pool.dim() != 4 or out.shape != q.shape:
        raise ValueError("bad tensor ranks or out shape")
    S, Hq, d = q.shape
    N, Hkv, B, d2 = k_pool.shape
    if d2 != d or tuple(v_pool.shape) != (N, Hkv, B, d):
        raise ValueError("k_pool and v_pool must both be [N][H_kv][B][d]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
        raise ValueError("block_tables must be [S][max_blocks] and context_lens [S]")
    if out.dtype not in (torch.float32, k_pool.dtype):
        raise TypeError("out must be float32 or the cache dtype")
    if workspace is None:
        workspace = decode_workspace(S, Hq, Hkv, d, num_workers, q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(L.paged_attn_decode(
        _dev(out, "out"), _DT[out.dtype], _dev(q, "q", k_pool.dtype), _dev(k_pool, "k_pool"),
        _dev(v_pool, "v_pool", k_pool.dtype), kdt, _dev(block_tables, "block_tables", torch.int32),
        int(block_tables.shape[1]), _dev(context_lens, "context_lens", torch.int32),
        int(max_context_len), S, Hq, Hkv, d, B, N, float(scale), int(num_workers), ws_ptr,
        ws_bytes, _stream(stream)))
    return out


def shared_prefix_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, prefix_len,
                            num_workers=0, device="cuda") -> torch.Tensor:
    """Allocate a workspace for paged_attn_decode_shared_prefix with these sizes."""
    n = int(load_library().pkv_shared_prefix_workspace_size(
        num_seqs, num_q_heads, num_kv_heads, head_dim, num_workers, prefix_len))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def paged_attn_decode_shared_prefix(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor,
                                    v_pool: torch.Tensor, prefix_blocks: torch.Tensor,
                                    prefix_len: int, block_tables: torch.Tensor,
                                    context_lens: torch.Tensor, max_context_len: int,
                                    scale: float = 0.0, num_workers: int = 0,
                                    workspace: Optional[torch.Tensor] = None,
                                    stream=None) -> torch.Tensor:
    """paged_attn_decode for sequences that all begin with the ``prefix_len`` tokens held in
    the shared blocks ``prefix_blocks`` (int32 [prefix_len / B]), which are read once for all of
    them (C: ``paged_attn_decode_shared_prefix``). Other arguments as paged_attn_decode."""
    L = load_library()
    kdt = _kv_dtype(k_pool)
    if q.dim() != 3 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape or out.shape != q.shape:
        raise ValueError("bad tensor ranks or out shape; k_pool and v_pool must match")
    S, Hq, d = q.shape
    N, Hkv, B, d2 = k_pool.shape
    if d2 != d:
        raise ValueError("head_dim of q and the pools differ")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
        raise ValueError("block_tables must be [S][max_blocks] and context_lens [S]")
    if prefix_blocks.dim() != 1 or prefix_blocks.shape[0] * B < int(prefix_len):
        raise ValueError("prefix_blocks must list the prefix_len / B shared blocks")
    if out.dtype not in (torch.float32, k_pool.dtype):
        raise TypeError("out must be float32 or the cache dtype")
    if workspace is None:
        workspace = shared_prefix_workspace(S, Hq, Hkv, d, prefix_len, num_workers, q.device)
    _check(L.paged_attn_decode_shared_prefix(
        _dev(out, "out"), _DT[out.dtype], _dev(q, "q", k_pool.dtype), _dev(k_pool, "k_pool"),
        _dev(v_pool, "v_pool", k_pool.dtype), kdt, _dev(prefix_blocks, "prefix_blocks", torch.int32),
        int(prefix_len), _dev(block_tables, "block_tables", torch.int32),
        int(block_tables.shape[1]), _dev(context_lens, "context_lens", torch.int32),
        int(max_context_len), S, Hq, Hkv, d, B, N, float(scale), int(num_workers),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


def extend_workspace(num_seqs, num_query_tokens, num_q_heads, num_kv_heads, head_dim,
                     max_query_len, max_context_len, device="cuda") -> torch.Tensor:
    """Allocate a workspace for paged_attn_extend with these sizes."""
    n = int(load_library().pkv_extend_workspace_size(num_seqs, num_query_tokens, num_q_heads,
                                                     num_kv_heads, head_dim, max_query_len,
                                                     max_context_len))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def paged_attn_extend(out: torch.Tensor, q: torch.Tensor, query_start: torch.Tensor,
                      max_query_len: int, k_pool: torch.Tensor, v_pool: torch.Tensor,
                      block_tables: torch.Tensor, context_lens: torch.Tensor,
                      max_context_len: int, scale: float = 0.0,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Causal attention of each sequence's new query tokens (rows query_start[s] ..
    query_start[s+1] - 1 of q, [T][H_q][d]) over its paged cache, whose last n_s tokens are the
    new ones (C: ``paged_attn_extend``)."""
    L = load_library()
    kdt = _kv_dtype(k_pool)
    if q.dim() != 3 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape or out.shape != q.shape:
        raise ValueError("bad tensor ranks or out shape; k_pool and v_pool must match")
    T, Hq, d = q.shape
    N, Hkv, B, d2 = k_pool.shape
    S = int(context_lens.shape[0])
    if d2 != d or tuple(query_start.shape) != (S + 1,) or block_tables.shape[0] != S:
        raise ValueError("query_start must be [S + 1], block_tables [S][max_blocks]")
    if out.dtype not in (torch.float32, k_pool.dtype):
        raise TypeError("out must be float32 or the cache dtype")
    if workspace is None:
        workspace = extend_workspace(S, T, Hq, Hkv, d, max_query_len, max_context_len, q.device)
    _check(L.paged_attn_extend(
        _dev(out, "out"), _DT[out.dtype], _dev(q, "q", k_pool.dtype),
        _dev(query_start, "query_start", torch.int32), T, int(max_query_len),
        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool", k_pool.dtype), kdt,
        _dev(block_tables, "block_tables", torch.int32), int(block_tables.shape[1]),
        _dev(context_lens, "context_lens", torch.int32), int(max_context_len), S, Hq, Hkv, d, B,
        N, float(scale), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


DECODE_STATIC_SCRATCH = 32 << 20   # bytes of the library's static decode scratch per GPU


def paged_attn_decode_noalloc(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor,
                              v_pool: torch.Tensor, block_tables: torch.Tensor,
                              context_lens: torch.Tensor, max_context_len: int,
                              scale: float = 0.0, num_workers: int = 0,
                              stream=None) -> torch.Tensor:
    """paged_attn_decode with the library's static scratch in place of a workspace (C:
    ``paged_attn_decode_noalloc``): nothing is allocated. Calls that overlap on one GPU race."""
    L = load_library()
    kdt = _kv_dtype(k_pool)
    if q.dim() != 3 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape or out.shape != q.shape:
        raise ValueError("bad tensor ranks or out shape; k_pool and v_pool must match")
    S, Hq, d = q.shape
    N, Hkv, B, d2 = k_pool.shape
    if d2 != d:
        raise ValueError("q and the pools disagree on head_dim")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
        raise ValueError("block_tables must be [S][max_blocks] and context_lens [S]")
    if out.dtype not in (torch.float32, k_pool.dtype):
        raise TypeError("out must be float32 or the cache dtype")
    _check(L.paged_attn_decode_noalloc(
        _dev(out, "out"), _DT[out.dtype], _dev(q, "q", k_pool.dtype), _dev(k_pool, "k_pool"),
        _dev(v_pool, "v_pool", k_pool.dtype), kdt, _dev(block_tables, "block_tables", torch.int32),
        int(block_tables.shape[1]), _dev(context_lens, "context_lens", torch.int32),
        int(max_context_len), S, Hq, Hkv, d, B, N, float(scale), int(num_workers),
        _stream(stream)))
    return out


def paged_attn_decode_append(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor,
                             v_pool: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                             block_tables: torch.Tensor, context_lens: torch.Tensor,
                             max_context_len: int, scale: float = 0.0, num_workers: int = 0,
                             workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Append k_new[s] / v_new[s] ([S][H_kv][d]) at position context_lens[s] - 1 and decode,
    in one call (C: ``paged_attn_decode_append``). Other arguments as paged_attn_decode."""
    L = load_library()
    kdt = _kv_dtype(k_pool)
    if q.dim() != 3 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape or out.shape != q.shape:
        raise ValueError("bad tensor ranks or out shape; k_pool and v_pool must match")
    S, Hq, d = q.shape
    N, Hkv, B, d2 = k_pool.shape
    if d2 != d or tuple(k_new.shape) != (S, Hkv, d) or tuple(v_new.shape) != (S, Hkv, d):
        raise ValueError("k_new/v_new must be [S][H_kv][d]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
        raise ValueError("block_tables must be [S][max_blocks] and context_lens [S]")
    if out.dtype not in (torch.float32, k_pool.dtype):
        raise TypeError("out must be float32 or the cache dtype")
    if workspace is None:
        workspace = decode_workspace(S, Hq, Hkv, d, num_workers, q.device)
    _check(L.paged_attn_decode_append(
        _dev(out, "out"), _DT[out.dtype], _dev(q, "q", k_pool.dtype), _dev(k_pool, "k_pool"),
        _dev(v_pool, "v_pool", k_pool.dtype), kdt, _dev(k_new, "k_new", k_pool.dtype),
        _dev(v_new, "v_new", k_pool.dtype), _dev(block_tables, "block_tables", torch.int32),
        int(block_tables.shape[1]), _dev(context_lens, "context_lens", torch.int32),
        int(max_context_len), S, Hq, Hkv, d, B, N, float(scale), int(num_workers),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


def kv_cache_append(k_pool, v_pool, k_new, v_new, seq_ids, positions, block_tables,
                    stream=None):
    """Store K/V rows of new tokens ([n][H_kv][d]) at their slots (C: ``kv_cache_append``)."""
    L = load_library()
    N, Hkv, B, d = k_pool.shape
    if v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool must both be [N][H_kv][B][d]")
    n = int(k_new.shape[0])
    if tuple(k_new.shape) != (n, Hkv, d) or tuple(v_new.shape) != (n, Hkv, d):
        raise ValueError("k_new/v_new must be [n][H_kv][d]")
    if tuple(seq_ids.shape) != (n,) or tuple(positions.shape) != (n,):
        raise ValueError("seq_ids/positions must be [n]")
    _check(L.kv_cache_append(
        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool", k_pool.dtype), _kv_dtype(k_pool),
        _dev(k_new, "k_new", k_pool.dtype), _dev(v_new, "v_new", k_pool.dtype),
        _dev(seq_ids, "seq_ids", torch.int32), _dev(positions, "positions", torch.int32), n,
        _dev(block_tables, "block_tables", torch.int32), int(block_tables.shape[1]),
        int(block_tables.shape[0]), Hkv, d, B, N, _stream(stream)))


def cow_block_copy(k_pool, v_pool, src_blocks, dst_blocks, num_tokens=None, stream=None):
    """Copy the first n slots of block src to block dst, all heads, K and V (C:
    ``cow_block_copy``). ``num_tokens`` None copies whole blocks."""
    L = load_library()
    N, Hkv, B, d = k_pool.shape
    if v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool must both be [N][H_kv][B][d]")
    n = int(src_blocks.shape[0])
    if tuple(dst_blocks.shape) != (n,) or (num_tokens is not None and tuple(num_tokens.shape) != (n,)):
        raise ValueError("src/dst/num_tokens must be [num_pairs]")
    nt = _dev(num_tokens, "num_tokens", torch.int32) if num_tokens is not None else None
    _check(L.cow_block_copy(
        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool", k_pool.dtype), _kv_dtype(k_pool),
        _dev(src_blocks, "src_blocks", torch.int32), _dev(dst_blocks, "dst_blocks", torch.int32),
        nt, n, Hkv, d, B, N, _stream(stream)))


def _host_pool(t: torch.Tensor, name: str, like: torch.Tensor) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.is_cuda or not t.is_pinned():
        raise ValueError(f"{name} must be a pinned host tensor (pin_memory=True)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != like.dtype or tuple(t.shape[1:]) != tuple(like.shape[1:]):
        raise ValueError(f"{name} must be [num_host_blocks]{list(like.shape[1:])} of {like.dtype}")
    return t.data_ptr()


def _swap(fn, k_pool, v_pool, host_k, host_v, first_ids, second_ids, stream):
    N, Hkv, B, d = k_pool.shape
    if v_pool.shape != k_pool.shape or host_v.shape != host_k.shape:
        raise ValueError("K and V pools must have equal shapes")
    n = int(first_ids.shape[0])
    if first_ids.dim() != 1 or tuple(second_ids.shape) != (n,):
        raise ValueError("block id lists must be [num_pairs]")
    _check(fn(_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool", k_pool.dtype), _kv_dtype(k_pool),
              _host_pool(host_k, "host_k", k_pool), _host_pool(host_v, "host_v", k_pool),
              int(host_k.shape[0]), _dev(first_ids, "block ids", torch.int32),
              _dev(second_ids, "block ids", torch.int32), n, Hkv, d, B, N, _stream(stream)))


def kv_swap_out(k_pool, v_pool, host_k, host_v, device_blocks, host_blocks, stream=None):
    """Copy whole blocks device_blocks[i] of the pools to host_blocks[i] of the pinned host
    pools (C: ``kv_swap_out``). Asynchronous: synchronize before reading the host pools."""
    _swap(load_library().kv_swap_out, k_pool, v_pool, host_k, host_v, device_blocks,
          host_blocks, stream)


def kv_swap_in(k_pool, v_pool, host_k, host_v, host_blocks, device_blocks, stream=None):
    """Copy whole blocks host_blocks[i] of the pinned host pools to device_blocks[i] of the
    pools (C: ``kv_swap_in``)."""
    _swap(load_library().kv_swap_in, k_pool, v_pool, host_k, host_v, host_blocks,
          device_blocks, stream)


def swap_staging(num_pairs: int, k_pool: torch.Tensor) -> torch.Tensor:
    """Staging buffer for the copy-engine swap of ``num_pairs`` blocks of ``k_pool``'s shape."""
    N, Hkv, B, d = k_pool.shape
    n = load_library().pkv_swap_staging_size(int(num_pairs), Hkv, d, B, _kv_dtype(k_pool))
    return torch.empty(max(int(n), 16), dtype=torch.uint8, device=k_pool.device)


def _swap_dma(fn, out, k_pool, v_pool, host_k, host_v, device_blocks, host_block0, staging,
              stream):
    N, Hkv, B, d = k_pool.shape
    if v_pool.shape != k_pool.shape or host_v.shape != host_k.shape:
        raise ValueError("K and V pools must have equal shapes")
    if device_blocks.dim() != 1:
        raise ValueError("device_blocks must be [num_pairs]")
    n = int(device_blocks.shape[0])
    hk, hv = _host_pool(host_k, "host_k", k_pool), _host_pool(host_v, "host_v", k_pool)
    ids = _dev(device_blocks, "device_blocks", torch.int32)
    st = _dev(staging, "staging", torch.uint8)
    nh = int(host_k.shape[0])
    if out:
        rc = fn(_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool", k_pool.dtype), _kv_dtype(k_pool),
                hk, hv, nh, ids, int(host_block0), n, Hkv, d, B, N, st, staging.numel(),
                _stream(stream))
    else:
        rc = fn(_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool", k_pool.dtype), _kv_dtype(k_pool),
                hk, hv, nh, int(host_block0), ids, n, Hkv, d, B, N, st, staging.numel(),
                _stream(stream))
    _check(rc)


def kv_swap_out_dma(k_pool, v_pool, host_k, host_v, device_blocks, host_block0, staging,
                    stream=None):
    """Copy blocks device_blocks[i] to host blocks host_block0 + i through ``staging`` and the
    copy engines (C: ``kv_swap_out_dma``)."""
    _swap_dma(load_library().kv_swap_out_dma, True, k_pool, v_pool, host_k, host_v,
              device_blocks, host_block0, staging, stream)


def kv_swap_in_dma(k_pool, v_pool, host_k, host_v, host_block0, device_blocks, staging,
                   stream=None):
    """Copy host blocks host_block0 + i to device_blocks[i] through ``staging`` and the copy
    engines (C: ``kv_swap_in_dma``)."""
    _swap_dma(load_library().kv_swap_in_dma, False, k_pool, v_pool, host_k, host_v,
              device_blocks, host_block0, staging, stream)


def stream_read_probe(src: torch.Tensor, sink: torch.Tensor, stream=None):
    """Read all of ``src`` once with plain 16-byte loads (C: ``pkv_stream_read_probe``)."""
    nbytes = src.numel() * src.element_size()
    _check(load_library().pkv_stream_read_probe(_dev(src, "src"), nbytes,
                                                _dev(sink, "sink", torch.int32), _stream(stream)))


def mfma_rate_probe(workgroups: int, iters: int, sink: torch.Tensor, stream=None):
    """workgroups x 4 wavefronts, each iters x 8 independent 16x16x32 bf16 MFMAs (C:
    ``pkv_mfma_rate_probe``)."""
    _check(load_library().pkv_mfma_rate_probe(int(workgroups), int(iters),
                                              _dev(sink, "sink", torch.float32), _stream(stream)))


def set_validate(on: bool = True):
    """Check device-resident contents (tables, lengths, slots) on the host before each call."""
    _check(load_library().pkv_set_validate(1 if on else 0))


def timing_enable(on=True, every: int = 1):
    """Time every ``every``-th launch of each library kernel (C: ``pkv_timing_enable``);
    ``on=False`` switches timing off."""
    _check(load_library().pkv_timing_enable(max(1, int(every)) if on else 0))


def timing_query(name: str = ""):
    """(total milliseconds, launches) of recorded kernels whose name contains ``name``."""
    tot = ctypes.c_double()
    n = ctypes.c_int64()
    _check(load_library().pkv_timing_query(name.encode(), ctypes.byref(tot), ctypes.byref(n)))
    return tot.value, n.value


class BlockPool:
    """Host block pool (C: ``pkv_pool_*`` and ``pkv_seq_*``). Table rows are int32 numpy
    arrays with -1 in unused entries."""

    def __init__(self, num_blocks: int):
        L = load_library()
        self._L = L
        self._p = L.pkv_pool_create(int(num_blocks))
        if not self._p:
            raise PagedKVError(-1, "pkv_pool_create failed")
        self.num_blocks = int(num_blocks)

    def __del__(self):
        p = getattr(self, "_p", None)
        if p:
            self._L.pkv_pool_destroy(p)
            self._p = None

    def alloc(self) -> int:
        b = ctypes.c_int32()
        rc = self._L.pkv_pool_alloc(self._p, ctypes.byref(b))
        if rc != 0:
            raise PagedKVError(rc, "pkv_pool_alloc")
        return b.value

    def claim(self, block: int):
        rc = self._L.pkv_pool_claim(self._p, int(block))
        if rc != 0:
            raise PagedKVError(rc, f"pkv_pool_claim({block})")

    def incref(self, block: int):
        rc = self._L.pkv_pool_incref(self._p, int(block))
        if rc != 0:
            raise PagedKVError(rc, f"pkv_pool_incref({block})")

    def decref(self, block: int) -> bool:
        f = ctypes.c_int()
        rc = self._L.pkv_pool_decref(self._p, int(block), ctypes.byref(f))
        if rc != 0:
            raise PagedKVError(rc, f"pkv_pool_decref({block})")
        return bool(f.value)

    def refcount(self, block: int) -> int:
        rc = self._L.pkv_pool_refcount(self._p, int(block))
        if rc < 0:
            raise PagedKVError(rc, f"pkv_pool_refcount({block})")
        return rc

    def num_free(self) -> int:
        return int(self._L.pkv_pool_num_free(self._p))

    @staticmethod
    def _row(row):
        import numpy as np
        if not (isinstance(row, np.ndarray) and row.dtype == np.int32 and row.flags.c_contiguous):
            raise TypeError("table rows must be contiguous int32 numpy arrays")
        return row.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))

    def prepare_write(self, row, length: int, block_size: int):
        """Returns (block, offset, cow) where cow is None or (src, dst, n)."""
        outs = [ctypes.c_int32() for _ in range(5)]
        rc = self._L.pkv_seq_prepare_write(self._p, self._row(row), int(row.shape[0]),
                                           int(length), int(block_size),
                                           *[ctypes.byref(o) for o in outs])
        if rc != 0:
            raise PagedKVError(rc, "pkv_seq_prepare_write")
        blk, off, cs, cd, cn = (o.value for o in outs)
        return blk, off, (None if cn < 0 else (cs, cd, cn))

    def fork(self, src_row, dst_row, num_blocks_used: int):
        rc = self._L.pkv_seq_fork(self._p, self._row(src_row), self._row(dst_row),
                                  int(num_blocks_used))
        if rc != 0:
            raise PagedKVError(rc, "pkv_seq_fork")

    def release(self, row, num_blocks_used: int) -> int:
        rc = self._L.pkv_seq_release(self._p, self._row(row), int(num_blocks_used))
        if rc < 0:
            raise PagedKVError(rc, "pkv_seq_release")
        return rc


class PrefixIndex:
    """Host prefix index over a BlockPool (C: ``pkv_prefix_index_*``): match the longest cached
    whole-block prefix of a token sequence, insert a computed sequence's blocks, evict least
    recently used unreferenced leaves."""

    def __init__(self, pool: "BlockPool", block_size: int):
        L = load_library()
        self._L = L
        self._pool = pool                     # kept alive: the index holds pool references
        self._x = L.pkv_prefix_index_create(pool._p, int(block_size))
        if not self._x:
            raise PagedKVError(-1, "pkv_prefix_index_create failed")
        self.block_size = int(block_size)

    def __del__(self):
        x = getattr(self, "_x", None)
        if x:
            self._L.pkv_prefix_index_destroy(x)
            self._x = None

    @staticmethod
    def _ints(values):
        import numpy as np
        a = np.ascontiguousarray(values, dtype=np.int32)
        return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))

    def match(self, tokens) -> list:
        t, tp = self._ints(tokens)
        cap = max(1, len(t) // self.block_size)
        out, op = self._ints([0] * cap)
        n = ctypes.c_int()
        _check(self._L.pkv_prefix_index_match(self._x, tp, len(t), op, cap, ctypes.byref(n)))
        return out[:n.value].tolist()

    def insert(self, tokens, blocks) -> int:
        t, tp = self._ints(tokens)
        b, bp = self._ints(blocks if len(blocks) else [0])
        n = ctypes.c_int()
        _check(self._L.pkv_prefix_index_insert(self._x, tp, len(t), bp, ctypes.byref(n)))
        return n.value

    def evict(self, max_blocks: int) -> list:
        out, op = self._ints([0] * max(1, int(max_blocks)))
        n = ctypes.c_int()
        _check(self._L.pkv_prefix_index_evict(self._x, int(max_blocks), op, ctypes.byref(n)))
        return out[:n.value].tolist()

    def size(self) -> int:
        return int(self._L.pkv_prefix_index_size(self._x))
