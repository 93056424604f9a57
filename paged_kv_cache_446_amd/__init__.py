"""MI355X-native paged KV cache and PagedAttention (gfx950).

The compute lives in ``libpkv.so`` (HIP kernels behind the C ABI of
``include/pkv.h``).  Submodules:

* ``ops``        kv_cache_write / paged_attention / copy_blocks on torch tensors
* ``allocator``  the reference-counted host block allocator
* ``build``      in-tree build of libpkv.so for gfx950

Importing ``ops`` or ``allocator`` loads the library and raises ImportError if
it has not been built; there is no CPU or Python fallback.
"""
