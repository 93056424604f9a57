"""Host checks of the metadata the kernels trust (calls into libpkv's plain-C checks).

Each function takes host (numpy) copies of the metadata a launch would get and
raises ``MetadataError`` naming the first offending entry; nothing touches a GPU.
``ops`` runs them before every launch when the environment sets ``PKV_DEBUG=1``.
"""

import ctypes

import numpy as np

from . import _lib


class MetadataError(ValueError):
    def __init__(self, what: str, index: int):
        self.index = index
        super().__init__(f"{what}: rule broken at index {index}" if index >= 0 else f"{what}: bad sizes")


def _p(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _call(name, *args):
    bad = ctypes.c_int32(-1)
    rc = getattr(_lib.load(), name)(*args, ctypes.byref(bad))
    if rc != _lib.PKV_OK:
        raise MetadataError(name, bad.value)


def slot_mapping(slots, num_blocks: int):
    """Every slot negative (padding) or below num_blocks * 16; no slot twice."""
    s = np.ascontiguousarray(slots, dtype=np.int64).ravel()
    _call("pkv_check_slot_mapping", _p(s, ctypes.c_int64), len(s), int(num_blocks))


def copy_pairs(pairs, num_blocks: int):
    """(src, dst) in the pool, src != dst, no dst twice, no dst that is also a src."""
    p = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    _call("pkv_check_copy_pairs", _p(p, ctypes.c_int32), len(p), int(num_blocks))


def batch(block_tables, seq_lens, query_start_loc, num_q_tokens: int, max_q_len: int,
          max_seq_len: int, num_blocks: int):
    """paged_attention's stated preconditions for every sequence of the batch."""
    t = np.ascontiguousarray(block_tables, dtype=np.int32)
    t = t.reshape(len(t), -1) if t.size else t.reshape(len(np.atleast_1d(seq_lens)), 0)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32).ravel()
    q = np.ascontiguousarray(query_start_loc, dtype=np.int32).ravel()
    if len(q) != len(sl) + 1 or len(t) != len(sl):
        raise MetadataError("pkv_check_batch", -1)
    _call("pkv_check_batch", _p(t, ctypes.c_int32), t.shape[1], _p(sl, ctypes.c_int32),
          _p(q, ctypes.c_int32), len(sl), int(num_q_tokens), int(max_q_len), int(max_seq_len),
          int(num_blocks))
