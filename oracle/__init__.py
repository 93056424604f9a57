"""CPU oracle for paged KV-cache attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct NumPy (fp64) and pure-Python code that states
what the hot path computes, written from the pages:

* blog.mckayzhao.com/?p=56, section "PagedAttention": KV cache split into
  16-token blocks located through a per-sequence block table; reading K/V block
  by block gives exactly the contiguous-storage result; N tokens need
  ceil(N/16) blocks, at most 15 slots wasted.
* same page, section on copy-on-write: reference-counted shared blocks; a
  sequence about to modify a shared block copies it first and leaves the
  original untouched.
* devpress.csdn.net/amd/6a408ab810ee7a33f2834f35.html, sections on prefill /
  decode (one KV entry appended per token), PagedAttention core idea (blocks
  handed out on demand from a free pool, returned when a request finishes) and
  sharing (several block tables pointing at one physical block).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, calls or links anything in here, and this
package never imports the product.  The two share only the seeded input
generators in ``workloads/``.

Every function here is pinned by ``-m "not gpu"`` tests (brute force on tiny
inputs, a library routine on the CPU, closed forms, invariants, and the
worked examples the pages print); nothing here is "parity unpinned".
"""

from . import numerics, layout, cache_ops, attention, allocator, brute  # noqa: F401
