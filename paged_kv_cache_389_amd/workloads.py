"""Seeded synthetic workloads for the paged decode path.

This module only draws random numbers and asks the host block manager for
block tables and slots.  It holds none of the attention or cache arithmetic,
so both the device path and the CPU oracle can be fed from it.

Five workload shapes (names used throughout the tests and the benchmark):

``tiny_fp32``
    4 sequences, 4 query heads = 4 KV heads, head_dim 64, block_size 16,
    context lengths uniform in [1, 64], a pool of 32 blocks handed out in a
    random order; scale 1/sqrt(64).
``opt13b_fp16``
    OPT-13B-shaped decode layer: 40 heads (MHA), head_dim 128, block_size 16,
    64 sequences, context lengths uniform in [128, 2048], blocks drawn at
    random from a pool of 8192.
``llama3_8b_gqa_bf16``
    Llama-3-8B-shaped GQA decode: 32 query / 8 KV heads, head_dim 128,
    block_size 16, 256 sequences, context lengths log-uniform in [16, 4096],
    random placement in a pool of 32768 blocks; each step first writes one new
    token per sequence through the slot mapping (the new token is the last
    of the ``L`` positions it then attends over).
``long_context_gqa_bf16``
    64 query / 8 KV heads, head_dim 128, block_size 32, 8 sequences, context
    lengths uniform in [16384, 32768], random placement in a pool of 12288
    blocks; 1% of key rows are multiplied by 8 after the cast.
``sharing_fp16``
    32 prompts, each forked into 8 sequences that share the prompt's blocks
    through reference counts, then diverge by 0-256 generated tokens; the
    first append into the shared partly filled last block triggers
    copy-on-write.  32 heads (MHA), head_dim 128, block_size 16, pool of 8192.
``llama3_8b_prefill_bf16``
    16 prompts of 512-2048 tokens whose every token is a query of the causal
    prefill attention; 32 query / 8 KV heads, head_dim 128, block_size 16,
    pool of 4096 blocks.
``system_prompt_bf16``
    128 distinct requests sharing 4 cached system prompts of 513-2047 tokens
    (last block partly filled; the cache entry keeps its own reference), each
    writing its own prompt of 16-512 tokens (its first token copies the
    shared partly filled block) and generating 0-64 tokens; 32 query / 8 KV
    heads, head_dim 128, block_size 16, pool of 8192 blocks.
``beam_search_fp16``
    16 requests with prompts of 256-1024 tokens, each decoded with 8 beams
    for 64 steps: every step appends one token to every beam (copy-on-write
    where beams share a partly filled last block), then each request's beams
    are re-drawn from their parents (forks of the chosen, frees of the
    dropped).  32 heads (MHA), head_dim 128, block_size 16, pool of 8192.

Values are N(0, 1) float32 draws cast (round to nearest even) to the
workload dtype.  Integer draws use numpy's PCG64 seeded with the workload
seed; tensor draws use a torch generator on the target device seeded with
the same seed, in the order q, K pool, V pool, key-outlier mask, new K, new V.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

from .block_manager import BlockManager

DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class DecodeStepInputs:
    """The integer and tensor inputs of one decode step's cache writes."""
    copy_pairs: np.ndarray          # int64 [n_pairs, 2]
    slot_mapping: np.ndarray        # int64 [n_tokens]
    seq_index: np.ndarray           # int64 [n_tokens], sequence of each token
    new_k: torch.Tensor | None = None   # [n_tokens, Hkv, hd]
    new_v: torch.Tensor | None = None
    # multi-step workloads whose batch changes between steps (beam search):
    # the tables and lengths the step's decode runs over, after its writes
    block_tables: np.ndarray | None = None   # int32 [n_seqs, W]
    context_lens: np.ndarray | None = None   # int32 [n_seqs]
    physical_blocks: int = 0                 # device blocks held after the step


@dataclass
class Workload:
    name: str
    dtype: torch.dtype
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    seed: int
    context_lens: np.ndarray        # int32 [B]
    block_tables: np.ndarray        # int32 [B, W]
    q: torch.Tensor                 # [B, Hq, hd]
    k_cache: torch.Tensor           # [num_blocks, Hkv, bs, hd]
    v_cache: torch.Tensor
    # the cache writes of the (last) step, applied before the attention
    step: DecodeStepInputs | None = None
    # multi-step history (sharing workload): every step's writes, in order
    history: list = field(default_factory=list)
    meta: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max(initial=0))

    @property
    def esize(self) -> int:
        return torch.tensor([], dtype=self.dtype).element_size()

    def kv_bytes(self) -> int:
        """K+V bytes the attention must read: each sequence's own context."""
        return int(self.context_lens.astype(np.int64).sum()) * 2 * \
            self.num_kv_heads * self.head_dim * self.esize

    def unique_kv_bytes(self) -> int:
        """K+V bytes of the distinct physical token slots referenced."""
        bs = self.block_size
        filled = {}
        for s in range(self.num_seqs):
            L = int(self.context_lens[s])
            for j in range((L + bs - 1) // bs):
                b = int(self.block_tables[s, j])
                filled[b] = max(filled.get(b, 0), min(bs, L - j * bs))
        return sum(filled.values()) * 2 * self.num_kv_heads * self.head_dim * self.esize

    def decode_bytes(self) -> int:
        """Algorithmic bytes of one decode call: K/V, q in, out, tables, lens."""
        bs = self.block_size
        nblk = int(((self.context_lens.astype(np.int64) + bs - 1) // bs).sum())
        qo = 2 * self.num_seqs * self.num_q_heads * self.head_dim * self.esize
        return self.kv_bytes() + qo + 4 * nblk + 4 * self.num_seqs

    def write_bytes(self) -> int:
        """Algorithmic bytes of the step's cache writes (read + write, K and V)."""
        if self.step is None:
            return 0
        row = self.num_kv_heads * self.head_dim * self.esize
        n_tok = len(self.step.slot_mapping)
        n_pair = len(self.step.copy_pairs)
        blk = row * self.block_size
        return 2 * (2 * n_tok * row) + 8 * n_tok + 2 * (2 * n_pair * blk) + 16 * n_pair


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, dtype, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dtype)


def _uniform_lens(lo, hi):
    def draw(rng, n):
        return rng.integers(lo, hi + 1, size=n)
    return draw


def _log_uniform_lens(lo, hi):
    def draw(rng, n):
        x = np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))
        return np.clip(np.rint(x), lo, hi).astype(np.int64)
    return draw


def build_decode(name, *, dtype, num_seqs, num_q_heads, num_kv_heads, head_dim,
                 block_size, num_blocks, lens, seed, device="cpu", scale=None,
                 key_outlier_frac=0.0, key_outlier_scale=8.0, new_token=False,
                 placement="random"):
    """A one-step decode workload (no sharing).

    ``lens`` is ``(lo, hi, "uniform"|"loguniform")`` or an explicit array.
    ``placement`` is ``"random"`` (a seeded permutation of the pool) or
    ``"sequential"`` (blocks handed out in increasing order; a control).
    """
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    rng = np.random.default_rng(seed)
    if isinstance(lens, tuple):
        lo, hi, kind = lens
        draw = _uniform_lens(lo, hi) if kind == "uniform" else _log_uniform_lens(lo, hi)
        context_lens = draw(rng, num_seqs).astype(np.int64)
    else:
        context_lens = np.asarray(lens, dtype=np.int64)
        assert len(context_lens) == num_seqs
    order = rng.permutation(num_blocks)
    if placement == "sequential":
        order = np.arange(num_blocks)[::-1]
    bm = BlockManager(num_blocks, block_size, free_order=order)
    seqs, slots = [], []
    for L in context_lens.tolist():
        s = bm.new_sequence()
        if new_token and L > 0:
            bm.extend(s, L - 1)
            slots.append(bm.append_slot(s))
        else:
            bm.extend(s, L)
        seqs.append(s)
    tables = bm.block_table_array(seqs, pad=0)
    g = _gen(device, seed)
    q = _randn((num_seqs, num_q_heads, head_dim), dt, g, device)
    pool_shape = (num_blocks, num_kv_heads, block_size, head_dim)
    k_cache = _randn(pool_shape, dt, g, device)
    v_cache = _randn(pool_shape, dt, g, device)
    if key_outlier_frac > 0:
        mask = torch.rand(pool_shape[:3], generator=g, device=device) < key_outlier_frac
        k_cache[mask] *= key_outlier_scale
    step = None
    if new_token:
        n = len(slots)
        step = DecodeStepInputs(
            copy_pairs=np.zeros((0, 2), np.int64),
            slot_mapping=np.asarray(slots, np.int64),
            seq_index=np.arange(num_seqs, dtype=np.int64)[context_lens > 0],
            new_k=_randn((n, num_kv_heads, head_dim), dt, g, device),
            new_v=_randn((n, num_kv_heads, head_dim), dt, g, device))
    return Workload(
        name=name, dtype=dt, num_seqs=num_seqs, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
        num_blocks=num_blocks,
        scale=(1.0 / math.sqrt(head_dim)) if scale is None else float(scale),
        seed=seed, context_lens=context_lens.astype(np.int32), block_tables=tables,
        q=q, k_cache=k_cache, v_cache=v_cache, step=step,
        meta={"placement": placement, "utilisation": bm.utilisation(seqs)})


def build_sharing(name="sharing_fp16", *, dtype="fp16", num_prompts=32, fanout=8,
                  prompt_len=1024, prompt_extra=(1, 15), max_gen=256,
                  num_heads=32, head_dim=128, block_size=16, num_blocks=8192,
                  seed=5, device="cpu", tensors=True):
    """Parallel-sampling workload with copy-on-write.

    Each prompt has ``prompt_len + r`` tokens already in the cache (``r``
    uniform in ``prompt_extra``: tokens the parent decoded before forking, so
    that the last shared block is partly filled).  The prompt is forked into
    ``fanout`` children holding every prompt block (count ``fanout``), and the
    parent's own hold is dropped.  Child ``c`` then appends ``d_c`` tokens,
    ``d_c`` uniform in [0, max_gen]; step ``t`` appends one token to every
    child with ``d_c >= t``, in sequence order.  ``history`` holds every step's
    copy pairs, slots and new rows; the decode runs over the final state.
    With ``prompt_extra=(0, 0)`` every shared block is full and no step copies.
    ``tensors=False`` skips every tensor draw (integer structure only).
    """
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    rng = np.random.default_rng(seed)
    lo, hi = prompt_extra
    extra = rng.integers(lo, hi + 1, size=num_prompts)
    gen = rng.integers(0, max_gen + 1, size=(num_prompts, fanout))
    bm = BlockManager(num_blocks, block_size, free_order=rng.permutation(num_blocks))
    children = []
    for p in range(num_prompts):
        parent = bm.new_sequence()
        bm.extend(parent, prompt_len + int(extra[p]))
        kids = [bm.fork(parent) for _ in range(fanout)]
        bm.free(parent)
        children.extend(kids)
    d = gen.reshape(-1)
    g = _gen(device, seed)
    num_seqs = num_prompts * fanout
    pool_shape = (num_blocks, num_heads, block_size, head_dim)
    q = k_cache = v_cache = None
    if tensors:
        q = _randn((num_seqs, num_heads, head_dim), dt, g, device)
        k_cache = _randn(pool_shape, dt, g, device)
        v_cache = _randn(pool_shape, dt, g, device)
    history = []
    for t in range(1, int(d.max(initial=0)) + 1):
        active = np.nonzero(d >= t)[0]
        slots = np.array([bm.append_slot(children[i]) for i in active], np.int64)
        pairs = bm.take_copy_pairs()
        st = DecodeStepInputs(copy_pairs=pairs, slot_mapping=slots,
                              seq_index=active.astype(np.int64))
        if tensors:
            st.new_k = _randn((len(slots), num_heads, head_dim), dt, g, device)
            st.new_v = _randn((len(slots), num_heads, head_dim), dt, g, device)
        history.append(st)
    tables = bm.block_table_array(children, pad=0)
    wl = Workload(
        name=name, dtype=dt, num_seqs=num_seqs, num_q_heads=num_heads,
        num_kv_heads=num_heads, head_dim=head_dim, block_size=block_size,
        num_blocks=num_blocks, scale=1.0 / math.sqrt(head_dim), seed=seed,
        context_lens=bm.context_lens(children), block_tables=tables, q=q,
        k_cache=k_cache, v_cache=v_cache,
        step=history[-1] if history else None, history=history,
        meta={"prompt_extra": extra, "gen": gen, "fanout": fanout,
              "prompt_len": prompt_len, "utilisation": bm.utilisation(children)})
    # copy-on-write pairs of the first step (the only step that copies)
    wl.meta["first_step_pairs"] = history[0].copy_pairs if history else np.zeros((0, 2), np.int64)
    return wl


def build_beam_search(name="beam_search_fp16", *, dtype="fp16", num_requests=16,
                      beam_width=8, prompt_lens=(256, 1024), steps=64, num_q_heads=32,
                      num_kv_heads=32, head_dim=128, block_size=16, num_blocks=8192,
                      selection_temp=2.0, seed=6, device="cpu", tensors=True):
    """Beam-search workload: repeated fork and free over shared prefixes.

    Each request's prompt (length uniform in ``prompt_lens``) is written once
    and forked into ``beam_width`` beams that hold all of its blocks; the
    prompt's own hold is dropped.  Step ``t`` (1..``steps``) appends one token
    to every beam, request by request, beam by beam; the block manager turns
    appends into shared partly filled blocks into copy-on-write pairs.  The
    step's decode runs over all beams after its writes.  Between steps each
    request re-draws its beams: every new beam picks a parent among the
    current ones with probability proportional to ``exp(selection_temp * z)``,
    ``z ~ N(0, 1)`` per current beam (a stand-in for the beams' scores);
    parents that nobody picked are freed, a parent picked ``c`` times is kept
    and forked ``c - 1`` times, and the new batch lists the beams parent by
    parent.  ``history`` holds every step's pairs, slots, new rows, and the
    tables and lengths its decode reads; the workload's own tables, lengths
    and ``q`` are those of the last step.  ``tensors=False`` skips every
    tensor draw (integer structure only).
    """
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    rng = np.random.default_rng(seed)
    lo, hi = prompt_lens
    plens = rng.integers(lo, hi + 1, size=num_requests)
    width = -(-(int(plens.max()) + steps) // block_size)
    bm = BlockManager(num_blocks, block_size, free_order=rng.permutation(num_blocks))
    beams = []                       # per request: its current beams, in batch order
    for r in range(num_requests):
        parent = bm.new_sequence()
        bm.extend(parent, int(plens[r]))
        beams.append([bm.fork(parent) for _ in range(beam_width)])
        bm.free(parent)
    num_seqs = num_requests * beam_width
    g = _gen(device, seed)
    pool_shape = (num_blocks, num_kv_heads, block_size, head_dim)
    k_cache = v_cache = None
    if tensors:
        k_cache = _randn(pool_shape, dt, g, device)
        v_cache = _randn(pool_shape, dt, g, device)
    history, lineage = [], []
    for t in range(1, steps + 1):
        batch = [b for req in beams for b in req]
        slots = np.array([bm.append_slot(b) for b in batch], np.int64)
        st = DecodeStepInputs(copy_pairs=bm.take_copy_pairs(), slot_mapping=slots,
                              seq_index=np.arange(num_seqs, dtype=np.int64),
                              block_tables=bm.block_table_array(batch, width=width),
                              context_lens=bm.context_lens(batch),
                              physical_blocks=bm.num_blocks - bm.num_free)
        if tensors:
            st.new_k = _randn((num_seqs, num_kv_heads, head_dim), dt, g, device)
            st.new_v = _randn((num_seqs, num_kv_heads, head_dim), dt, g, device)
        history.append(st)
        if t == steps:
            break
        # re-draw the beams of every request from their parents
        parents_of_step = []
        for r in range(num_requests):
            z = rng.standard_normal(beam_width)
            w = np.exp(selection_temp * (z - z.max()))
            picks = rng.choice(beam_width, size=beam_width, p=w / w.sum())
            count = np.bincount(picks, minlength=beam_width)
            old = beams[r]
            for i in range(beam_width):
                if count[i] == 0:
                    bm.free(old[i])
            new, par = [], []
            for i in range(beam_width):
                if count[i]:
                    new.append(old[i])
                    new.extend(bm.fork(old[i]) for _ in range(count[i] - 1))
                    par.extend([r * beam_width + i] * int(count[i]))
            beams[r] = new
            parents_of_step.extend(par)
        lineage.append(np.array(parents_of_step, np.int64))
    final = history[-1]
    q = _randn((num_seqs, num_q_heads, head_dim), dt, g, device) if tensors else None
    wl = Workload(
        name=name, dtype=dt, num_seqs=num_seqs, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
        num_blocks=num_blocks, scale=1.0 / math.sqrt(head_dim), seed=seed,
        context_lens=final.context_lens, block_tables=final.block_tables, q=q,
        k_cache=k_cache, v_cache=v_cache, step=final, history=history,
        meta={"prompt_lens": plens, "beam_width": beam_width, "steps": steps,
              "parents": lineage, "utilisation": bm.utilisation([b for q_ in beams for b in q_])})
    return wl


def build_system_prompt(name="system_prompt_bf16", *, dtype="bf16", num_prefixes=4,
                        requests_per_prefix=32, prefix_blocks=(32, 127), prefix_extra=(1, 15),
                        own_prompt=(16, 512), max_gen=64, num_q_heads=32, num_kv_heads=8,
                        head_dim=128, block_size=16, num_blocks=8192, seed=8, device="cpu",
                        tensors=True):
    """Distinct requests that share a cached system prompt.

    Each of ``num_prefixes`` system prompts holds ``bs * k + r`` tokens (``k``
    uniform in ``prefix_blocks``, ``r`` uniform in ``prefix_extra``: with
    ``r > 0`` its last block is partly filled), written once into a cache
    entry that keeps its own reference to the prompt's blocks.  Requests
    arrive round-robin over the prompts (request i uses prompt i mod P):
    each forks its prompt's entry and writes its own prompt of ``n_i``
    tokens (uniform in ``own_prompt``), so its first token lands in the
    shared partly filled block and copies it (the entry still holds it);
    this admission step's copy-on-write pairs and slots are ``history[0]``.
    Request i then generates ``d_i`` tokens (uniform in [0, max_gen]); step
    t appends one token to every request with ``d_i >= t``.  The decode runs
    over the requests' final state (the cache entries are not in the batch).
    ``tensors=False`` skips every tensor draw (integer structure only).
    """
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    rng = np.random.default_rng(seed)
    bs = block_size
    plens = bs * rng.integers(prefix_blocks[0], prefix_blocks[1] + 1, size=num_prefixes) + \
        rng.integers(prefix_extra[0], prefix_extra[1] + 1, size=num_prefixes)
    num_seqs = num_prefixes * requests_per_prefix
    own = rng.integers(own_prompt[0], own_prompt[1] + 1, size=num_seqs)
    gen = rng.integers(0, max_gen + 1, size=num_seqs)
    bm = BlockManager(num_blocks, bs, free_order=rng.permutation(num_blocks))
    entries = []
    for p in range(num_prefixes):
        e = bm.new_sequence()
        bm.extend(e, int(plens[p]))
        entries.append(e)
    prefix_of = np.arange(num_seqs) % num_prefixes
    g = _gen(device, seed)
    pool_shape = (num_blocks, num_kv_heads, bs, head_dim)
    q = k_cache = v_cache = None
    if tensors:
        q = _randn((num_seqs, num_q_heads, head_dim), dt, g, device)
        k_cache = _randn(pool_shape, dt, g, device)
        v_cache = _randn(pool_shape, dt, g, device)
    reqs, slots, seq_index = [], [], []
    for i in range(num_seqs):
        x = bm.fork(entries[prefix_of[i]])
        slots.append(bm.extend(x, int(own[i])))
        seq_index.append(np.full(int(own[i]), i, np.int64))
        reqs.append(x)
    admit = DecodeStepInputs(copy_pairs=bm.take_copy_pairs(),
                             slot_mapping=np.concatenate(slots).astype(np.int64),
                             seq_index=np.concatenate(seq_index))
    history = [admit]
    for t in range(1, int(gen.max(initial=0)) + 1):
        active = np.nonzero(gen >= t)[0]
        st = DecodeStepInputs(copy_pairs=np.zeros((0, 2), np.int64),
                              slot_mapping=np.array([bm.append_slot(reqs[i]) for i in active],
                                                    np.int64),
                              seq_index=active.astype(np.int64))
        pairs = bm.take_copy_pairs()
        assert len(pairs) == 0, "generation appends into blocks the request owns"
        history.append(st)
    if tensors:
        for st in history:
            n = len(st.slot_mapping)
            st.new_k = _randn((n, num_kv_heads, head_dim), dt, g, device)
            st.new_v = _randn((n, num_kv_heads, head_dim), dt, g, device)
    wl = Workload(
        name=name, dtype=dt, num_seqs=num_seqs, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=bs, num_blocks=num_blocks,
        scale=1.0 / math.sqrt(head_dim), seed=seed, context_lens=bm.context_lens(reqs),
        block_tables=bm.block_table_array(reqs, pad=0), q=q, k_cache=k_cache, v_cache=v_cache,
        step=history[-1], history=history,
        meta={"prefix_lens": plens, "prefix_of": prefix_of, "own_prompt": own, "gen": gen,
              "entry_tables": [list(e.table) for e in entries],
              "refcount": bm.refcount.copy(), "physical_blocks": bm.num_blocks - bm.num_free,
              "utilisation": bm.utilisation(reqs + entries)})
    wl.meta["first_step_pairs"] = admit.copy_pairs
    return wl


@dataclass
class PrefillWorkload:
    """Causal multi-token attention inputs: sequence s has ``context_lens[s]``
    cached tokens, of which the last ``query_start[s+1] - query_start[s]`` are
    queries (rows of ``q``)."""
    name: str
    dtype: torch.dtype
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    seed: int
    context_lens: np.ndarray        # int32 [B]
    query_start: np.ndarray         # int32 [B + 1]
    block_tables: np.ndarray        # int32 [B, W]
    q: torch.Tensor                 # [total_q, Hq, hd]
    k_cache: torch.Tensor
    v_cache: torch.Tensor

    @property
    def total_q(self) -> int:
        return int(self.query_start[-1])

    @property
    def max_q_len(self) -> int:
        return int(np.diff(self.query_start).max(initial=0))

    @property
    def esize(self) -> int:
        return torch.tensor([], dtype=self.dtype).element_size()

    def flops(self) -> int:
        """Causal attention flops: 4 * hd per (query row, head, visible token)
        (QK and PV, one multiply-add = 2 flops each)."""
        vis = 0
        for s in range(self.num_seqs):
            n = int(self.query_start[s + 1] - self.query_start[s])
            L = int(self.context_lens[s])
            p = np.arange(L - n, L)
            vis += int(np.clip(p + 1, 0, None).sum())
        return 4 * self.head_dim * self.num_q_heads * vis

    def min_bytes(self) -> int:
        """Bytes the call must move at least: every visible K/V row once, q
        in, out."""
        kv = int(self.context_lens.astype(np.int64).sum()) * 2 * self.num_kv_heads * \
            self.head_dim * self.esize
        return kv + 2 * self.total_q * self.num_q_heads * self.head_dim * self.esize


def build_prefill(name, *, dtype, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                  num_blocks, lens, chunk=None, seed, device="cpu"):
    """Prefill workload: contexts of ``lens`` (``(lo, hi)`` uniform or an
    array) in randomly placed blocks; each sequence's queries are its last
    ``min(L, chunk)`` positions (all of them when ``chunk`` is None)."""
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    rng = np.random.default_rng(seed)
    if isinstance(lens, tuple):
        context_lens = rng.integers(lens[0], lens[1] + 1, size=num_seqs)
    else:
        context_lens = np.asarray(lens, dtype=np.int64)
    bm = BlockManager(num_blocks, block_size, free_order=rng.permutation(num_blocks))
    seqs = []
    for L in context_lens.tolist():
        sq = bm.new_sequence()
        bm.extend(sq, L)
        seqs.append(sq)
    nq = context_lens if chunk is None else np.minimum(context_lens, chunk)
    query_start = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    g = _gen(device, seed)
    pool_shape = (num_blocks, num_kv_heads, block_size, head_dim)
    q = _randn((int(query_start[-1]), num_q_heads, head_dim), dt, g, device)
    k_cache = _randn(pool_shape, dt, g, device)
    v_cache = _randn(pool_shape, dt, g, device)
    return PrefillWorkload(
        name=name, dtype=dt, num_seqs=num_seqs, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
        num_blocks=num_blocks, scale=1.0 / math.sqrt(head_dim), seed=seed,
        context_lens=context_lens.astype(np.int32), query_start=query_start,
        block_tables=bm.block_table_array(seqs, pad=0), q=q, k_cache=k_cache, v_cache=v_cache)


def llama3_8b_prefill_bf16(seed=7, device="cpu", **kw):
    """Llama-3-8B-shaped prefill: 16 prompts of 512-2048 tokens, every token a
    query (32 query / 8 KV heads, head_dim 128, block_size 16)."""
    args = dict(dtype="bf16", num_seqs=16, num_q_heads=32, num_kv_heads=8, head_dim=128,
                block_size=16, num_blocks=4096, lens=(512, 2048))
    args.update(kw)
    return build_prefill("llama3_8b_prefill_bf16", seed=seed, device=device, **args)


def sharing_saving(wl, step=None) -> float:
    """1 - physical / logical blocks of a multi-step workload's step (default:
    the last): the share of block memory that sharing saves against giving
    every sequence its own copy of its blocks."""
    st = wl.history[-1] if step is None else wl.history[step]
    logical = int(((st.context_lens.astype(np.int64) + wl.block_size - 1) // wl.block_size).sum())
    return 1.0 - st.physical_blocks / logical if logical else 0.0


# Full-size presets -------------------------------------------------------

def tiny_fp32(seed=1, device="cpu", **kw):
    args = dict(dtype="fp32", num_seqs=4, num_q_heads=4, num_kv_heads=4, head_dim=64,
                block_size=16, num_blocks=32, lens=(1, 64, "uniform"), scale=1.0 / 8.0)
    args.update(kw)
    return build_decode("tiny_fp32", seed=seed, device=device, **args)


def opt13b_fp16(seed=2, device="cpu", **kw):
    args = dict(dtype="fp16", num_seqs=64, num_q_heads=40, num_kv_heads=40, head_dim=128,
                block_size=16, num_blocks=8192, lens=(128, 2048, "uniform"))
    args.update(kw)
    return build_decode("opt13b_fp16", seed=seed, device=device, **args)


def llama3_8b_gqa_bf16(seed=3, device="cpu", **kw):
    args = dict(dtype="bf16", num_seqs=256, num_q_heads=32, num_kv_heads=8, head_dim=128,
                block_size=16, num_blocks=32768, lens=(16, 4096, "loguniform"),
                new_token=True)
    args.update(kw)
    return build_decode("llama3_8b_gqa_bf16", seed=seed, device=device, **args)


def long_context_gqa_bf16(seed=4, device="cpu", **kw):
    args = dict(dtype="bf16", num_seqs=8, num_q_heads=64, num_kv_heads=8, head_dim=128,
                block_size=32, num_blocks=12288, lens=(16384, 32768, "uniform"),
                key_outlier_frac=0.01)
    args.update(kw)
    return build_decode("long_context_gqa_bf16", seed=seed, device=device, **args)


def sharing_fp16(seed=5, device="cpu", **kw):
    return build_sharing("sharing_fp16", seed=seed, device=device, **kw)


def beam_search_fp16(seed=6, device="cpu", **kw):
    return build_beam_search("beam_search_fp16", seed=seed, device=device, **kw)


def system_prompt_bf16(seed=8, device="cpu", **kw):
    return build_system_prompt("system_prompt_bf16", seed=seed, device=device, **kw)


WORKLOADS = {
    "tiny_fp32": tiny_fp32,
    "opt13b_fp16": opt13b_fp16,
    "llama3_8b_gqa_bf16": llama3_8b_gqa_bf16,
    "long_context_gqa_bf16": long_context_gqa_bf16,
    "sharing_fp16": sharing_fp16,
    "beam_search_fp16": beam_search_fp16,
    "system_prompt_bf16": system_prompt_bf16,
    "llama3_8b_prefill_bf16": llama3_8b_prefill_bf16,
}


def make(name, **kw) -> Workload:
    return WORKLOADS[name](**kw)
