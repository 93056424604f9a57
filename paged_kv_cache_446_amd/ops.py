"""Device entry points over torch tensors: argument marshalling only.

Every step runs in libpkv's HIP kernels; torch provides device memory and the
current stream.  Tensors of element type bf16/fp16/fp32 may also be passed as
raw-bit views (int16 / int32) together with an explicit ``dtype``.
"""

import ctypes
import os

import torch

from . import _lib, checks

_lib.load()  # no fallback: importing the binding without the HIP library fails here

# PKV_DEBUG=1: copy each launch's metadata to the host and check it first (slow; synchronizes)
DEBUG = os.environ.get("PKV_DEBUG", "0") not in ("", "0")

_TORCH_DTYPES = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


class PagedCache:
    """K and V block pools [num_layers][num_blocks][num_kv_heads][16 * head_dim]."""

    def __init__(self, k_pool: torch.Tensor, v_pool: torch.Tensor, num_kv_heads: int, head_dim: int,
                 dtype: str = None, num_layers: int = 1):
        dtype = dtype or _TORCH_DTYPES[k_pool.dtype]
        assert k_pool.is_cuda and v_pool.is_cuda and k_pool.is_contiguous() and v_pool.is_contiguous()
        self.k_pool, self.v_pool = k_pool, v_pool
        self.dtype = dtype
        self.num_layers = num_layers
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        elem = {"f32": 4, "f16": 2, "bf16": 2}[dtype]
        per_block = num_kv_heads * 16 * head_dim * elem
        nbytes = k_pool.numel() * k_pool.element_size()
        assert nbytes % (per_block * num_layers) == 0 and nbytes == v_pool.numel() * v_pool.element_size()
        self.num_blocks = nbytes // (per_block * num_layers)
        self.desc = _lib.CacheDesc(k_pool.data_ptr(), v_pool.data_ptr(), num_layers, self.num_blocks,
                                   num_kv_heads, head_dim, _lib.DTYPE_CODES[dtype])
        lib = _lib.load()
        assert lib.pkv_pool_bytes(ctypes.byref(self.desc)) == nbytes


def kv_cache_write(cache: PagedCache, k_new, v_new, slot_mapping, layer: int = 0, stream=None):
    lib = _lib.load()
    assert slot_mapping.dtype == torch.int64 and slot_mapping.is_contiguous()
    assert k_new.is_contiguous() and v_new.is_contiguous()
    T = slot_mapping.numel()
    if DEBUG:
        checks.slot_mapping(slot_mapping.cpu().numpy(), cache.num_blocks)
    _lib.check(lib.pkv_kv_cache_write(ctypes.byref(cache.desc), layer, _ptr(k_new), _ptr(v_new),
                                      _ptr(slot_mapping), T, _stream(stream)), "pkv_kv_cache_write")


def copy_blocks(cache: PagedCache, pairs, stream=None):
    lib = _lib.load()
    assert pairs.dtype == torch.int32 and pairs.is_contiguous()
    n = pairs.numel() // 2
    if DEBUG:
        checks.copy_pairs(pairs.cpu().numpy(), cache.num_blocks)
    _lib.check(lib.pkv_copy_blocks(ctypes.byref(cache.desc), _ptr(pairs) if n else None, n,
                                   _stream(stream)), "pkv_copy_blocks")


def workspace_bytes(num_seqs, num_q_tokens, max_seq_len, num_q_heads, head_dim) -> int:
    return int(_lib.load().pkv_paged_attention_workspace_bytes(num_seqs, num_q_tokens, max_seq_len,
                                                               num_q_heads, head_dim))


def paged_attention(cache: PagedCache, out, q, block_tables, seq_lens, query_start_loc, *,
                    num_q_heads: int, max_q_len: int, max_seq_len: int, scale: float,
                    workspace, layer: int = 0, shared_prefixes: bool = False, stream=None):
    """shared_prefixes: rows share prefixes of blocks (a speed hint; results are the
    same either way)."""
    lib = _lib.load()
    for t, dt in ((block_tables, torch.int32), (seq_lens, torch.int32), (query_start_loc, torch.int32)):
        assert t.dtype == dt and t.is_contiguous() and t.is_cuda
    assert q.is_contiguous() and out.is_contiguous()
    S = seq_lens.numel()
    Tq = q.numel() // (num_q_heads * cache.head_dim)
    if DEBUG:
        checks.batch(block_tables.cpu().numpy(), seq_lens.cpu().numpy(), query_start_loc.cpu().numpy(),
                     Tq, max_q_len, max_seq_len, cache.num_blocks)
    _lib.check(lib.pkv_paged_attention(ctypes.byref(cache.desc), layer, _ptr(out), _ptr(q),
                                       _ptr(block_tables), block_tables.shape[-1], _ptr(seq_lens),
                                       _ptr(query_start_loc), S, Tq, max_q_len, max_seq_len,
                                       num_q_heads, float(scale), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(),
                                       1 if shared_prefixes else 0, _stream(stream)),
               "pkv_paged_attention")


def paged_attention_no_alloc(cache: PagedCache, out, q, block_tables, seq_lens, query_start_loc, *,
                             num_q_heads: int, max_q_len: int, max_seq_len: int, scale: float,
                             layer: int = 0, shared_prefixes: bool = False, stream=None):
    """paged_attention with the library's static per-GPU workspace (no allocation)."""
    lib = _lib.load()
    for t, dt in ((block_tables, torch.int32), (seq_lens, torch.int32), (query_start_loc, torch.int32)):
        assert t.dtype == dt and t.is_contiguous() and t.is_cuda
    assert q.is_contiguous() and out.is_contiguous()
    S = seq_lens.numel()
    Tq = q.numel() // (num_q_heads * cache.head_dim)
    if DEBUG:
        checks.batch(block_tables.cpu().numpy(), seq_lens.cpu().numpy(), query_start_loc.cpu().numpy(),
                     Tq, max_q_len, max_seq_len, cache.num_blocks)
    _lib.check(lib.pkv_paged_attention_no_alloc(ctypes.byref(cache.desc), layer, _ptr(out), _ptr(q),
                                                _ptr(block_tables), block_tables.shape[-1],
                                                _ptr(seq_lens), _ptr(query_start_loc), S, Tq,
                                                max_q_len, max_seq_len, num_q_heads, float(scale),
                                                1 if shared_prefixes else 0, _stream(stream)),
               "pkv_paged_attention_no_alloc")


def contiguous_attention(cache: PagedCache, out, q, first_block, seq_lens, query_start_loc, *,
                         num_q_heads: int, max_seq_len: int, scale: float, workspace, layer: int = 0,
                         stream=None):
    """Decode attention over sequences stored as contiguous block runs (no block table)."""
    lib = _lib.load()
    for t in (first_block, seq_lens, query_start_loc):
        assert t.dtype == torch.int32 and t.is_contiguous() and t.is_cuda
    assert q.is_contiguous() and out.is_contiguous()
    S = seq_lens.numel()
    Tq = q.numel() // (num_q_heads * cache.head_dim)
    _lib.check(lib.pkv_contiguous_attention(ctypes.byref(cache.desc), layer, _ptr(out), _ptr(q),
                                            _ptr(first_block), _ptr(seq_lens), _ptr(query_start_loc),
                                            S, Tq, max_seq_len, num_q_heads, float(scale),
                                            _ptr(workspace), workspace.numel() * workspace.element_size(),
                                            _stream(stream)), "pkv_contiguous_attention")


def calib_stream_read(buf, sink, stream=None):
    """Measurement only: read all of `buf` (a device tensor, size a multiple of 16
    bytes) once as a plain stream; `sink` is a 16-byte device tensor it may write."""
    lib = _lib.load()
    assert buf.is_contiguous() and sink.numel() * sink.element_size() >= 16
    _lib.check(lib.pkv_calib_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                         _stream(stream)), "pkv_calib_stream_read")
