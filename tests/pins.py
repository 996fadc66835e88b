"""Pins for the decode oracle: checks against things other than the oracle.

Each ``pin_*`` takes a batch decode function with the signature of
``oracle.decode`` and raises ``AssertionError`` when it disagrees with:

* a library attention routine (torch ``scaled_dot_product_attention`` in
  float64) on the contiguous keys and values, before paging;
* closed forms (one token, identical keys, zero scale, a hand-worked fixture);
* invariants (placement permutation, block size, key shift, linearity in V,
  NaN in every slot the sequence does not own, duplicated KV heads).

The paging used here is written independently of the oracle: a sequence's
contiguous ``[L, Hkv, hd]`` rows are padded to whole blocks, reshaped to
``[n_blocks, block_size, Hkv, hd]``, transposed to the cache layout and
stored at the table's physical blocks in one vectorised assignment.

``tests/test_oracle_mutants.py`` plants mistakes into copies of the oracle
and checks that these pins catch every one.
"""

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

TIGHT = 1e-12


def page(ks, vs, block_size, num_blocks, rng, poison=True, trap=True):
    """Lay contiguous per-sequence rows into a randomly placed block pool.

    Returns ``(k_pool, v_pool, tables, lens, perm)``.  Slots no sequence owns
    (unreferenced blocks, the tail of each last block) hold NaN when
    ``poison``; table entries past a sequence's blocks point at a trap block
    that is all NaN when ``trap``.
    """
    hkv, hd = ks[0].shape[1:]
    lens = np.array([k.shape[0] for k in ks], dtype=np.int64)
    nbs = [(int(L) + block_size - 1) // block_size for L in lens]
    need = sum(nbs) + 1
    assert need <= num_blocks, "pool too small"
    perm = rng.permutation(num_blocks)
    fill = np.nan if poison else 0.0
    kp = np.full((num_blocks, hkv, block_size, hd), fill)
    vp = np.full((num_blocks, hkv, block_size, hd), fill)
    trap_block = int(perm[-1])
    width = max(nbs) + 2
    tables = np.full((len(ks), width), trap_block if trap else 0, dtype=np.int64)
    used = 0
    for s, (k, v) in enumerate(zip(ks, vs)):
        nb = nbs[s]
        blocks = perm[used:used + nb]
        used += nb
        tables[s, :nb] = blocks
        for src, dst in ((k, kp), (v, vp)):
            padded = np.full((nb * block_size, hkv, hd), fill)
            padded[:src.shape[0]] = src
            dst[blocks] = padded.reshape(nb, block_size, hkv, hd).transpose(0, 2, 1, 3)
    return kp, vp, tables, lens, perm


def random_case(rng, num_seqs, hq, hkv, hd, lens, block_size=4, extra_blocks=3):
    q = rng.standard_normal((num_seqs, hq, hd))
    ks = [rng.standard_normal((int(L), hkv, hd)) for L in lens]
    vs = [rng.standard_normal((int(L), hkv, hd)) for L in lens]
    nblk = sum((int(L) + block_size - 1) // block_size for L in lens) + extra_blocks
    return q, ks, vs, nblk


def sdpa_reference(q, ks, vs, scale):
    """Contiguous attention by the library routine, float64, per sequence."""
    out = np.zeros(q.shape)
    for s in range(q.shape[0]):
        L = ks[s].shape[0]
        if L == 0:
            continue
        Q = torch.from_numpy(q[s]).double()[None, :, None, :]
        K = torch.from_numpy(ks[s]).double().permute(1, 0, 2)[None].contiguous()
        V = torch.from_numpy(vs[s]).double().permute(1, 0, 2)[None].contiguous()
        o = F.scaled_dot_product_attention(Q, K, V, scale=scale,
                                           enable_gqa=Q.shape[1] != K.shape[1])
        out[s] = o[0, :, 0, :].numpy()
    return out


def _run(decode, q, kp, vp, tables, lens, scale, hkv):
    return np.asarray(decode(q, kp, vp, tables, lens, scale, hkv), dtype=np.float64)


# --------------------------------------------------------------------- pins

def pin_brute_force(decode, seed=0):
    """Paged oracle == library attention on contiguous data (MHA and GQA,
    several block sizes, partial tails, single tokens)."""
    rng = np.random.default_rng(seed)
    shapes = [  # (num_seqs, hq, hkv, hd, lens, block_size)
        (3, 2, 2, 8, [1, 5, 9], 4),
        (2, 4, 1, 6, [7, 16], 4),
        (4, 6, 2, 4, [3, 8, 13, 2], 8),
        (2, 8, 4, 16, [33, 17], 16),
    ]
    for (b, hq, hkv, hd, lens, bs) in shapes:
        q, ks, vs, nblk = random_case(rng, b, hq, hkv, hd, lens, bs)
        scale = 1.0 / math.sqrt(hd)
        kp, vp, tables, L, _ = page(ks, vs, bs, nblk, rng)
        got = _run(decode, q, kp, vp, tables, L, scale, hkv)
        ref = sdpa_reference(q, ks, vs, scale)
        err = np.abs(got - ref).max()
        assert err <= TIGHT, f"brute force {b, hq, hkv, hd, lens, bs}: max err {err}"


def pin_permutation_invariance(decode, seed=1):
    """Moving blocks to other physical places (and rewriting the tables)
    leaves the result bit-identical."""
    rng = np.random.default_rng(seed)
    q, ks, vs, nblk = random_case(rng, 3, 4, 2, 8, [6, 11, 4], 4, extra_blocks=6)
    r1 = _run(decode, q, *page(ks, vs, 4, nblk, rng)[:4], 0.3, 2)
    r2 = _run(decode, q, *page(ks, vs, 4, nblk, rng)[:4], 0.3, 2)
    assert np.array_equal(r1, r2), "placement changed the result"


def pin_single_token(decode, seed=2):
    """One token: the output is that token's value row, exactly."""
    rng = np.random.default_rng(seed)
    q, ks, vs, nblk = random_case(rng, 2, 4, 2, 8, [1, 1], 4)
    kp, vp, tables, L, _ = page(ks, vs, 4, nblk, rng)
    got = _run(decode, q, kp, vp, tables, L, 0.7, 2)
    for s in range(2):
        for h in range(4):
            assert np.array_equal(got[s, h], vs[s][0, h // 2]), "L=1 is not the value row"


def pin_uniform_weights(decode, seed=3):
    """Identical keys, or a zero scale: the output is the mean value row."""
    rng = np.random.default_rng(seed)
    q, ks, vs, nblk = random_case(rng, 2, 2, 2, 8, [7, 12], 4)
    same = [np.broadcast_to(k[:1], k.shape).copy() for k in ks]
    for keys, scale in ((same, 0.5), (ks, 0.0)):
        kp, vp, tables, L, _ = page(keys, vs, 4, nblk, rng)
        got = _run(decode, q, kp, vp, tables, L, scale, 2)
        for s in range(2):
            want = vs[s].mean(axis=0)
            assert np.abs(got[s] - want).max() <= TIGHT, "uniform weights != mean"


def pin_poison(decode, seed=4):
    """Slots a sequence does not own never reach the result: NaN there
    changes nothing (compare against the same case with zeros there)."""
    rng = np.random.default_rng(seed)
    q, ks, vs, nblk = random_case(rng, 3, 2, 1, 8, [5, 9, 3], 4, extra_blocks=4)
    state = rng.bit_generator.state
    a = _run(decode, q, *page(ks, vs, 4, nblk, rng, poison=True, trap=True)[:4], 0.4, 1)
    rng.bit_generator.state = state
    b = _run(decode, q, *page(ks, vs, 4, nblk, rng, poison=False, trap=False)[:4], 0.4, 1)
    assert np.all(np.isfinite(a)), "poisoned slots leaked into the result"
    assert np.array_equal(a, b), "unowned slots changed the result"


def pin_gqa_duplication(decode, seed=5):
    """Grouped heads == the same run with every KV head copied ``group``
    times (MHA), bit for bit."""
    rng = np.random.default_rng(seed)
    hq, hkv = 6, 2
    g = hq // hkv
    q, ks, vs, nblk = random_case(rng, 2, hq, hkv, 8, [6, 10], 4)
    state = rng.bit_generator.state
    a = _run(decode, q, *page(ks, vs, 4, nblk, rng)[:4], 0.35, hkv)
    ks_m = [np.repeat(k, g, axis=1) for k in ks]
    vs_m = [np.repeat(v, g, axis=1) for v in vs]
    rng.bit_generator.state = state
    b = _run(decode, q, *page(ks_m, vs_m, 4, nblk, rng)[:4], 0.35, hq)
    assert np.array_equal(a, b), "GQA differs from duplicated-head MHA"


def pin_block_size_invariance(decode, seed=6):
    """The same logical sequence paged at block sizes 2, 4 and 8 gives the
    same result."""
    rng = np.random.default_rng(seed)
    q, ks, vs, _ = random_case(rng, 2, 2, 2, 8, [9, 14], 4)
    res = []
    for bs in (2, 4, 8):
        nblk = sum((k.shape[0] + bs - 1) // bs for k in ks) + 3
        res.append(_run(decode, q, *page(ks, vs, bs, nblk, rng)[:4], 0.3, 2))
    for r in res[1:]:
        assert np.abs(r - res[0]).max() <= TIGHT, "block size changed the result"


def pin_shift_invariance(decode, seed=7):
    """Adding one vector c to every key (scale * q.c = 1000) leaves the
    softmax unchanged; a version without the max subtraction overflows."""
    rng = np.random.default_rng(seed)
    q, ks, vs, nblk = random_case(rng, 1, 1, 1, 8, [12], 4)
    scale = 0.25
    c = q[0, 0] / np.dot(q[0, 0], q[0, 0]) * (1000.0 / scale)
    shifted = [k + c for k in ks]
    state = rng.bit_generator.state
    a = _run(decode, q, *page(ks, vs, 4, nblk, rng)[:4], scale, 1)
    rng.bit_generator.state = state
    b = _run(decode, q, *page(shifted, vs, 4, nblk, rng)[:4], scale, 1)
    assert np.all(np.isfinite(b)), "large scores overflowed"
    assert np.abs(a - b).max() <= 1e-9, "shift of the keys changed the result"


def pin_linearity_in_values(decode, seed=8):
    """out(alpha*V1 + V2) == alpha*out(V1) + out(V2) for fixed keys."""
    rng = np.random.default_rng(seed)
    q, ks, v1, nblk = random_case(rng, 2, 2, 2, 8, [7, 10], 4)
    v2 = [rng.standard_normal(v.shape) for v in v1]
    alpha = -1.75
    mix = [alpha * a + b for a, b in zip(v1, v2)]
    outs = []
    for vs in (v1, v2, mix):
        r = np.random.default_rng(99)
        outs.append(_run(decode, q, *page(ks, vs, 4, nblk, r)[:4], 0.3, 2))
    assert np.abs(outs[2] - (alpha * outs[0] + outs[1])).max() <= 1e-11, "not linear in V"


def pin_golden_three_tokens(decode, golden_dir):
    """Hand-worked paged example: weights 1/8, 2/8, 5/8 -> (6, 7)."""
    with open(os.path.join(golden_dir, "paged_softmax_three_tokens.json")) as f:
        g = json.load(f)
    bs, nb = g["block_size"], g["num_blocks"]
    hd = len(g["q"])
    kp = np.full((nb, 1, bs, hd), np.nan)
    vp = np.full((nb, 1, bs, hd), np.nan)
    for tok in g["tokens"]:
        kp[tok["block"], 0, tok["offset"]] = tok["k"]
        vp[tok["block"], 0, tok["offset"]] = tok["v"]
    q = np.array(g["q"], dtype=np.float64)[None, None, :]
    tables = np.array([g["block_table"] + [1, 1]], dtype=np.int64)
    lens = np.array([g["context_len"]])
    got = _run(decode, q, kp, vp, tables, lens, g["scale"], 1)[0, 0]
    assert np.abs(got - np.array(g["expected_out"])).max() <= g["abs_tol"], got


ALL_DECODE_PINS = [
    pin_brute_force, pin_permutation_invariance, pin_single_token,
    pin_uniform_weights, pin_poison, pin_gqa_duplication,
    pin_block_size_invariance, pin_shift_invariance, pin_linearity_in_values,
]
