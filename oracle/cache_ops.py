"""Oracle: the cache-writing operations, applied to host arrays in place.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Both operations move bytes and do no arithmetic on them, so the GPU results
must match these byte for byte over the whole cache buffer.  Callers pass
integer views of the caches (``int16`` for 16-bit floats, ``int32`` for
float32) so that NaN payloads and signed zeros are compared as bits.

Cache layout: ``[num_blocks, num_kv_heads, block_size, head_dim]``.
"""

import numpy as np


def reshape_and_cache(k, v, k_cache, v_cache, slot_mapping):
    """Write each new token's key and value rows into its cache slot.

    A new token is written into the slot the block manager gave it: slot
    ``b * block_size + o`` is offset ``o`` of physical block ``b``.  Blocks are
    filled as generation proceeds ("Memory Optimization in LLM Serving with
    PagedAttention", section "How PagedAttention Works", on-demand allocation;
    "vLLM and PagedAttention ...", paragraph on the solution), and after a
    copy-on-write the write lands in the new copy (section "Advanced
    Capabilities: Memory Sharing with Copy-on-Write").  The slot convention
    and the skip of negative slots are readings; the pages do not fix them.

    ``k`` and ``v`` are ``[num_tokens, num_kv_heads, head_dim]``.
    """
    block_size = k_cache.shape[2]
    for j, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        block, offset = divmod(int(slot), block_size)
        k_cache[block, :, offset, :] = k[j]
        v_cache[block, :, offset, :] = v[j]


def copy_blocks(k_cache, v_cache, src_dst_pairs):
    """Copy whole physical blocks: ``cache[dst] = cache[src]`` for K and V.

    This is the copy step of copy-on-write: before a sequence appends to a
    block that other sequences also reference, the content of that block is
    copied into a freshly allocated block ("Memory Optimization in LLM Serving
    with PagedAttention", section "Advanced Capabilities: Memory Sharing with
    Copy-on-Write"); only that one block is copied, not the whole cache
    ("vLLM and PagedAttention ...", paragraph on sharing).
    """
    for src, dst in np.asarray(src_dst_pairs).reshape(-1, 2).tolist():
        k_cache[int(dst)] = k_cache[int(src)]
        v_cache[int(dst)] = v_cache[int(src)]


def swap_blocks(src_k, src_v, dst_k, dst_v, src_dst_pairs):
    """Move whole blocks between two pools: ``dst[dst_i] = src[src_i]`` for K
    and V.

    When memory runs short the engine evicts whole sequences by swapping
    their blocks out to CPU memory, and brings them back later ("vLLM and
    PagedAttention: How Ideas from Operating Systems Accelerated LLM
    Inference", paragraph on the engine).  Either pool may be the device
    cache; the copy is of bytes only.
    """
    for src, dst in np.asarray(src_dst_pairs).reshape(-1, 2).tolist():
        dst_k[int(dst)] = src_k[int(src)]
        dst_v[int(dst)] = src_v[int(src)]
