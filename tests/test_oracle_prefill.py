"""Pins of the prefill oracle (no GPU): torch's causal
scaled_dot_product_attention on contiguous data, the decode oracle for one
query per sequence, chunk invariance (a chunk of queries gives the rows a
full prefill gives for the same positions), placement invariance, a
hand-worked causal case, and zero rows for queries before the context."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import pins


def _case(rng, lens, hq, hkv, hd, bs):
    ks = [rng.standard_normal((L, hkv, hd)) for L in lens]
    vs = [rng.standard_normal((L, hkv, hd)) for L in lens]
    nblk = sum(-(-L // bs) for L in lens) + 3
    kp, vp, tables, cl, _ = pins.page(ks, vs, bs, nblk, rng)
    return ks, vs, kp, vp, tables, cl


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2)])
def test_full_prefill_matches_torch_causal_sdpa(hq, hkv):
    """Every token of every sequence is a query (n == L): the library's
    causal attention on the contiguous rows (top-left and bottom-right
    alignment coincide for a square mask)."""
    rng = np.random.default_rng(40 + hq)
    lens = [1, 5, 16, 23]
    ks, vs, kp, vp, tables, cl = _case(rng, lens, hq, hkv, 8, 4)
    qs = np.concatenate([[0], np.cumsum(lens)])
    q = rng.standard_normal((int(qs[-1]), hq, 8))
    got = oracle.prefill(q, kp, vp, tables, cl, qs, 0.37, hkv)
    for s, L in enumerate(lens):
        Q = torch.from_numpy(q[qs[s]:qs[s + 1]]).permute(1, 0, 2)[None].contiguous()
        K = torch.from_numpy(ks[s]).permute(1, 0, 2)[None].contiguous()
        V = torch.from_numpy(vs[s]).permute(1, 0, 2)[None].contiguous()
        want = F.scaled_dot_product_attention(Q, K, V, scale=0.37, is_causal=True,
                                              enable_gqa=hq != hkv)[0].permute(1, 0, 2)
        assert np.allclose(got[qs[s]:qs[s + 1]], want.numpy(), rtol=0, atol=1e-12)


def test_chunk_rows_equal_full_prefill_rows():
    """Queries for the last n positions only (chunked prefill / recompute of
    a suffix) give the same rows as the full prefill's last n rows."""
    rng = np.random.default_rng(50)
    lens = [9, 30]
    _, _, kp, vp, tables, cl = _case(rng, lens, 4, 2, 8, 8)
    qs_full = np.array([0, 9, 39])
    q_full = rng.standard_normal((39, 4, 8))
    full = oracle.prefill(q_full, kp, vp, tables, cl, qs_full, 0.5, 2)
    n = [3, 11]
    qs = np.array([0, 3, 14])
    q = np.concatenate([q_full[9 - 3:9], q_full[39 - 11:39]])
    part = oracle.prefill(q, kp, vp, tables, cl, qs, 0.5, 2)
    assert np.array_equal(part, np.concatenate([full[6:9], full[28:39]]))


def test_one_query_per_sequence_is_decode():
    rng = np.random.default_rng(51)
    lens = [1, 7, 20]
    _, _, kp, vp, tables, cl = _case(rng, lens, 4, 1, 8, 4)
    q = rng.standard_normal((3, 4, 8))
    got = oracle.prefill(q, kp, vp, tables, cl, np.arange(4), 0.3, 1)
    assert np.array_equal(got, oracle.decode(q, kp, vp, tables, cl, 0.3, 1))


def test_placement_permutation_invariance():
    rng = np.random.default_rng(52)
    lens = [13, 6]
    ks, vs, kp, vp, tables, cl = _case(rng, lens, 2, 2, 8, 4)
    qs = np.array([0, 5, 11])
    q = rng.standard_normal((11, 2, 8))
    a = oracle.prefill(q, kp, vp, tables, cl, qs, 0.4, 2)
    kp2, vp2, tables2, _, _ = pins.page(ks, vs, 4, kp.shape[0], np.random.default_rng(99))
    b = oracle.prefill(q, kp2, vp2, tables2, cl, qs, 0.4, 2)
    assert np.allclose(a, b, rtol=0, atol=1e-13)


def test_hand_worked_causal_case():
    """One head, head_dim 1, keys 0, 1, 2, values 10, 20, 30, q = 1, scale 1,
    all three tokens queried: row 0 sees token 0 (10); row 1 sees tokens 0-1
    with weights e^0, e^1; row 2 sees all three with e^0, e^1, e^2."""
    kp = np.array([[[[0.0], [1.0], [2.0], [np.nan]]]])
    vp = np.array([[[[10.0], [20.0], [30.0], [np.nan]]]])
    q = np.ones((3, 1, 1))
    got = oracle.prefill(q, kp, vp, np.array([[0]]), np.array([3]), np.array([0, 3]), 1.0, 1)
    e = np.e
    want = [10.0, (10 + 20 * e) / (1 + e), (10 + 20 * e + 30 * e * e) / (1 + e + e * e)]
    assert np.allclose(got[:, 0, 0], want, rtol=0, atol=1e-12)


def test_queries_before_the_context_are_zero_rows():
    """n > L: the first n - L queries sit before position 0 and see nothing."""
    rng = np.random.default_rng(53)
    _, _, kp, vp, tables, cl = _case(rng, [2], 2, 2, 4, 4)
    q = rng.standard_normal((5, 2, 4))
    got = oracle.prefill(q, kp, vp, tables, cl, np.array([0, 5]), 0.5, 2)
    assert np.array_equal(got[:3], np.zeros((3, 2, 4)))
    assert np.isfinite(got[3:]).all()
