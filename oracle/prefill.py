"""Oracle: multi-token (prefill / recompute) causal attention over a paged KV
cache, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages give: when memory runs short the engine evicts whole
sequences and later brings them back by swapping or by recomputation ("vLLM
and PagedAttention: How Ideas from Operating Systems Accelerated LLM
Inference", paragraph on the engine); recomputation runs the sequence's
tokens through the model again, that is, attention of many query tokens at
once over the same paged cache.  The pages print no formula, so the reading
is the plainest one that fits the decode path:

* sequence s has ``L = context_lens[s]`` tokens in the cache (the new ones
  included, written beforehand) and ``n = query_start[s+1] - query_start[s]``
  query tokens, which are its LAST n positions: query i sits at position
  ``p = L - n + i``;
* query i attends causally to cache positions ``0 .. p`` (the ``p + 1``
  first tokens), through the block table exactly as decode does; a query
  with ``p < 0`` (more queries than tokens) attends to nothing and gives a
  zero row;
* one query row is therefore decode attention with context length
  ``p + 1``: this oracle is that definition, row by row, on ``decode_one``.

Layouts: ``q`` and the result are ``[total_q, num_q_heads, head_dim]``
(sequence s owns rows ``query_start[s] .. query_start[s+1]``); the caches and
tables are those of ``decode``.
"""

import numpy as np

from .paged_attention import decode_one, kv_head_of


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, num_kv_heads,
            rows=None, heads=None):
    """Causal paged attention of every query row (float64).  ``rows`` /
    ``heads`` restrict the work to a sample; other rows are left NaN."""
    total, num_q_heads, head_dim = q.shape
    qs = np.asarray(query_start, dtype=np.int64)
    out = np.full((total, num_q_heads, head_dim), np.nan)
    seq_of = np.zeros(total, dtype=np.int64)
    for s in range(len(qs) - 1):
        seq_of[qs[s]:qs[s + 1]] = s
    rows = range(total) if rows is None else rows
    heads = range(num_q_heads) if heads is None else heads
    for r in rows:
        s = int(seq_of[r])
        n = int(qs[s + 1] - qs[s])
        L = int(context_lens[s])
        p = L - n + (r - int(qs[s]))
        for h in heads:
            if p < 0:
                out[r, h] = 0.0
                continue
            out[r, h] = decode_one(q[r, h], k_cache, v_cache, block_tables[s], p + 1, scale,
                                   kv_head_of(h, num_q_heads, num_kv_heads))
    return out
