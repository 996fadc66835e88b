"""Oracle: single-query (decode) attention over a paged KV cache, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed
----------------
The pages say the PagedAttention kernel gathers a sequence's scattered KV
blocks and then performs the attention calculation as usual ("Memory
Optimization in LLM Serving with PagedAttention", section "How PagedAttention
Works"; "vLLM and PagedAttention ...", paragraph on the engine).  Paging
changes where keys and values live, not the result.  So this oracle is the
plain definition, written out:

* a sequence's cache is a run of logical blocks of ``block_size`` tokens;
  logical block ``j`` lives in the physical block ``block_table[j]`` (same
  page, "How PagedAttention Works", items 1-3);
* only the last block may be partly filled, so a sequence of ``L`` tokens
  uses ``ceil(L / block_size)`` table entries and token ``t`` sits in logical
  block ``t // block_size`` at offset ``t % block_size`` (same section, the
  bullet on fragmentation; "vLLM and PagedAttention ...", paragraph on the
  solution);
* the attention formula itself is not printed on the pages.  Reading taken:
  standard scaled dot-product attention of one query row against the
  sequence's ``L`` keys, softmax over those ``L`` scores, weighted sum of the
  ``L`` value rows.  With grouped query heads (not on the pages either), query
  head ``h`` reads KV head ``h // (num_q_heads // num_kv_heads)``.
* ``L == 0`` gives a zero row (reading taken; no workload produces it).

Cache layout: ``k_cache`` and ``v_cache`` are ``[num_blocks, num_kv_heads,
block_size, head_dim]``.  Inputs may be numpy arrays or CPU torch tensors of
any float dtype; values are upcast exactly to float64 before any arithmetic.
The result is left unrounded in float64.
"""

import numpy as np

try:  # torch is optional for the oracle; used only to upcast bf16 tensors.
    import torch as _torch
except Exception:  # pragma: no cover - torch is present in this image
    _torch = None


def _f64(x):
    """Exact upcast of a numpy array or CPU torch tensor to a float64 array."""
    if _torch is not None and isinstance(x, _torch.Tensor):
        return x.detach().to("cpu", _torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def kv_head_of(q_head, num_q_heads, num_kv_heads):
    """KV head read by query head ``q_head`` (consecutive grouping; a reading,
    since grouped-query attention is not on the pages)."""
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    return q_head // (num_q_heads // num_kv_heads)


def decode_one(q_row, k_cache, v_cache, table_row, context_len, scale, kv_head):
    """Attention output (float64, shape [head_dim]) of one query row.

    The sequence's keys and values are looked up logical block by logical
    block through ``table_row``; the last block contributes only its first
    ``L - j * block_size`` slots.
    """
    q = _f64(q_row)
    head_dim = q.shape[0]
    L = int(context_len)
    if L == 0:
        return np.zeros(head_dim)
    block_size = k_cache.shape[2]
    n_logical = -(-L // block_size)
    scores = np.empty(L)
    values = np.empty((L, head_dim))
    for j in range(n_logical):
        phys = int(table_row[j])
        first = j * block_size
        used = min(block_size, L - first)
        k_rows = _f64(k_cache[phys, kv_head, :used, :])
        v_rows = _f64(v_cache[phys, kv_head, :used, :])
        scores[first:first + used] = scale * (k_rows @ q)
        values[first:first + used] = v_rows
    # softmax with the maximum subtracted first, so large scores cannot overflow
    weights = np.exp(scores - scores.max())
    return (weights @ values) / weights.sum()


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, num_kv_heads,
           seqs=None, heads=None):
    """Paged decode attention for a batch: ``out[s, h] = decode_one(...)``.

    ``q`` is ``[num_seqs, num_q_heads, head_dim]``; ``block_tables`` is
    ``[num_seqs, max_blocks]`` (entries past ``ceil(L / block_size)`` are never
    read); ``context_lens`` is ``[num_seqs]``.  ``seqs`` / ``heads`` restrict
    the work to a sample; other rows of the result are left NaN.
    """
    num_seqs, num_q_heads, head_dim = q.shape
    out = np.full((num_seqs, num_q_heads, head_dim), np.nan)
    seqs = range(num_seqs) if seqs is None else seqs
    heads = range(num_q_heads) if heads is None else heads
    for s in seqs:
        for h in heads:
            out[s, h] = decode_one(q[s, h], k_cache, v_cache, block_tables[s],
                                   context_lens[s], scale,
                                   kv_head_of(h, num_q_heads, num_kv_heads))
    return out
