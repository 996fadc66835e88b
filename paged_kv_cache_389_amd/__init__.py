"""MI355X-native paged KV-cache decode path.

Device calls (hand-written gfx950 HIP kernels behind the C ABI in
``include/pagedkv.h``; the Python names are the C names without ``pkv_``):

* :func:`paged_attention_decode` - single-query attention over a KV cache kept
  in fixed-size physical blocks reached through per-sequence block tables;
* :func:`reshape_and_cache` - write new tokens' K/V rows into their slots;
* :func:`copy_blocks` - copy whole blocks (the copy of copy-on-write);
* :func:`swap_blocks` - move whole blocks between the device cache and a
  pool in pinned host memory (eviction by swapping);
* :func:`reshape_and_cache_fp8`, :func:`paged_attention_decode_fp8` - the
  same write and attention over an 8-bit (OCP E4M3) cache with per-cache
  scales;
* :func:`paged_attention_prefill` - causal attention of many query tokens per
  sequence over the paged cache (prefill / recomputation);
* :func:`paged_attention_decode_grouped` - decode of sequences that share
  blocks (forks of one prompt), each shared tile read once per group.

Host side: :mod:`.block_manager` (block pool, tables, reference counts, fork,
copy-on-write) and :mod:`.workloads` (seeded synthetic inputs).

The device calls load ``libpagedkv.so`` on first use and raise
:class:`NativeLibraryMissing` if it is not built; nothing falls back to a
CPU implementation.
"""

_NATIVE = ("paged_attention_decode", "reshape_and_cache", "copy_blocks", "swap_blocks",
           "reshape_and_cache_fp8", "paged_attention_decode_fp8", "KV_E4M3",
           "paged_attention_prefill", "paged_attention_decode_grouped", "grouped_workspace_bytes",
           "group_tiles",
           "workspace_bytes", "plan",
           "version", "NativeLibraryMissing", "PagedKVError", "PATH_AUTO", "PATH_VALU",
           "PATH_MFMA", "PATH_CONTIGUOUS", "PATH_SHARED_BLOCKS", "GRID_AUTO", "GRID_DIRECT", "GRID_PLANNED", "HipEvent")

__all__ = list(_NATIVE) + ["block_manager", "workloads"]


def __getattr__(name):
    if name in _NATIVE:
        from . import _native
        return getattr(_native, name)
    raise AttributeError(name)
