"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle.

Bars: bit-exact for reshape_and_cache and copy_blocks (whole cache buffers);
max-abs error <= 1e-5 (fp32) or 2e-2 (fp16 / bf16, fp32 accumulation)
against the unrounded float64 oracle for attention.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import pins
from gpu_helpers import (DEV, INT_VIEW, TOL, decode_gpu, max_err, say, upload_case)
from paged_kv_cache_389_amd import _native as pk

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.float16, torch.bfloat16]
DT_ID = {torch.float32: "fp32", torch.float16: "fp16", torch.bfloat16: "bf16"}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")


def _rand_bits(shape, dtype, gen):
    """Random bit patterns (any value, NaN payloads included)."""
    iv = INT_VIEW[dtype]
    info = torch.iinfo(iv)
    return torch.randint(info.min, info.max, shape, generator=gen, dtype=torch.int64).to(iv)


# ------------------------------------------------------------- copy_blocks

@pytest.mark.parametrize("dtype", DTYPES, ids=DT_ID.get)
def test_copy_blocks_bit_exact(dtype):
    say("copy_blocks", DT_ID[dtype])
    g = torch.Generator().manual_seed(101)
    nb, hkv, bs, hd = 64, 4, 16, 128
    kbits = _rand_bits((nb, hkv, bs, hd), dtype, g)
    vbits = _rand_bits((nb, hkv, bs, hd), dtype, g)
    pairs = np.array([[3, 40], [7, 41], [3, 42], [63, 0], [10, 11]], np.int64)
    kd, vd = kbits.to(DEV).view(dtype), vbits.to(DEV).view(dtype)
    from paged_kv_cache_389_amd import copy_blocks
    copy_blocks(kd, vd, torch.from_numpy(pairs).to(DEV))
    torch.cuda.synchronize()
    ko, vo = kbits.numpy().copy(), vbits.numpy().copy()
    oracle.copy_blocks(ko, vo, pairs)
    assert np.array_equal(kd.view(INT_VIEW[dtype]).cpu().numpy(), ko)
    assert np.array_equal(vd.view(INT_VIEW[dtype]).cpu().numpy(), vo)


def test_copy_blocks_many_pairs_and_odd_block_bytes():
    """More pairs than fit one launch's grid dimension is not needed here;
    a block whose byte size is not a multiple of the 16 KiB chunk is."""
    say("copy_blocks odd size")
    g = torch.Generator().manual_seed(102)
    nb, hkv, bs, hd = 300, 3, 8, 64       # 3*8*64*2 = 3072-byte blocks
    kbits = _rand_bits((nb, hkv, bs, hd), torch.float16, g)
    vbits = _rand_bits((nb, hkv, bs, hd), torch.float16, g)
    rng = np.random.default_rng(5)
    perm = rng.permutation(nb)
    pairs = np.stack([perm[:100], perm[100:200]], axis=1).astype(np.int64)
    kd, vd = kbits.to(DEV).view(torch.float16), vbits.to(DEV).view(torch.float16)
    from paged_kv_cache_389_amd import copy_blocks
    copy_blocks(kd, vd, torch.from_numpy(pairs).to(DEV))
    torch.cuda.synchronize()
    ko, vo = kbits.numpy().copy(), vbits.numpy().copy()
    oracle.copy_blocks(ko, vo, pairs)
    assert np.array_equal(kd.view(torch.int16).cpu().numpy(), ko)
    assert np.array_equal(vd.view(torch.int16).cpu().numpy(), vo)


def test_copy_blocks_skips_out_of_range_pairs():
    say("copy_blocks out of range")
    g = torch.Generator().manual_seed(103)
    kbits = _rand_bits((8, 2, 16, 64), torch.float16, g)
    kd = kbits.to(DEV).view(torch.float16)
    vd = kd.clone()
    before = kd.clone()
    from paged_kv_cache_389_amd import copy_blocks
    copy_blocks(kd, vd, torch.tensor([[-1, 2], [3, 8], [9, 1]], dtype=torch.int64, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(kd.view(torch.int16), before.view(torch.int16))


# ------------------------------------------------------- reshape_and_cache

@pytest.mark.parametrize("dtype", DTYPES, ids=DT_ID.get)
@pytest.mark.parametrize("hd,bs", [(64, 16), (128, 16), (128, 32), (256, 8)])
def test_reshape_and_cache_bit_exact(dtype, hd, bs):
    say("reshape_and_cache", DT_ID[dtype], hd, bs)
    g = torch.Generator().manual_seed(201 + hd + bs)
    nb, hkv, ntok = 40, 4, 77
    kbits = _rand_bits((nb, hkv, bs, hd), dtype, g)
    vbits = _rand_bits((nb, hkv, bs, hd), dtype, g)
    newk = _rand_bits((ntok, hkv, hd), dtype, g)
    newv = _rand_bits((ntok, hkv, hd), dtype, g)
    rng = np.random.default_rng(hd * bs)
    slots = rng.choice(nb * bs, ntok, replace=False).astype(np.int64)
    slots[::7] = -1                                   # padding tokens
    kd, vd = kbits.to(DEV).view(dtype), vbits.to(DEV).view(dtype)
    from paged_kv_cache_389_amd import reshape_and_cache
    reshape_and_cache(newk.to(DEV).view(dtype), newv.to(DEV).view(dtype), kd, vd,
                      torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    ko, vo = kbits.numpy().copy(), vbits.numpy().copy()
    oracle.reshape_and_cache(newk.numpy(), newv.numpy(), ko, vo, slots)
    assert np.array_equal(kd.view(INT_VIEW[dtype]).cpu().numpy(), ko)
    assert np.array_equal(vd.view(INT_VIEW[dtype]).cpu().numpy(), vo)


def test_reshape_and_cache_skips_slots_past_the_pool():
    say("reshape_and_cache out of range")
    kd = torch.zeros(4, 2, 16, 64, dtype=torch.float16, device=DEV)
    vd = kd.clone()
    new = torch.ones(2, 2, 64, dtype=torch.float16, device=DEV)
    from paged_kv_cache_389_amd import reshape_and_cache
    reshape_and_cache(new, new, kd, vd, torch.tensor([64, 10**9], dtype=torch.int64, device=DEV))
    torch.cuda.synchronize()
    assert not kd.any() and not vd.any()


# ------------------------------------------------------------------ decode

def _case(seed, lens, hq, hkv, hd, bs, extra_blocks=5, poison=True):
    rng = np.random.default_rng(seed)
    q, ks, vs, nblk = pins.random_case(rng, len(lens), hq, hkv, hd, lens, bs, extra_blocks)
    kp, vp, tables, L, _ = pins.page(ks, vs, bs, nblk, rng, poison=poison)
    return q, kp, vp, tables, L


def _check_decode(q, kp, vp, tables, L, hkv, dtype, scale, partition=0, path=0, grid=0,
                  tol=None):
    dev, (qt, kt, vt) = upload_case(q, kp, vp, tables, L, dtype)
    got = decode_gpu(dev["q"], dev["k"], dev["v"], dev["tables"], dev["lens"], scale,
                     partition=partition, path=path, grid=grid)
    want = oracle.decode(qt, kt, vt, tables, L, scale, hkv)
    err = max_err(got, want)
    assert err <= (TOL[dtype] if tol is None else tol), f"max abs err {err}"
    return got, want


SHAPES = [  # (hq, hkv, hd, bs)
    (4, 4, 64, 16), (4, 4, 128, 16), (2, 2, 256, 32), (3, 3, 128, 8),
    (8, 2, 128, 16), (8, 1, 64, 32), (16, 2, 128, 32), (32, 2, 128, 16), (6, 3, 128, 16),
]


GRIDS = {"direct": 1, "planned": 2}


@pytest.mark.parametrize("grid", GRIDS.values(), ids=GRIDS.keys())
@pytest.mark.parametrize("dtype", DTYPES, ids=DT_ID.get)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "hq%d_hkv%d_hd%d_bs%d" % s)
def test_decode_ragged_lengths(dtype, shape, grid):
    hq, hkv, hd, bs = shape
    say("decode ragged", DT_ID[dtype], shape, grid)
    lens = [1, bs - 1, bs, bs + 1, 63, 64, 65, 200]
    q, kp, vp, tables, L = _case(7 + hd + bs + hq, lens, hq, hkv, hd, bs)
    _check_decode(q, kp, vp, tables, L, hkv, dtype, 1.0 / math.sqrt(hd), grid=grid)


@pytest.mark.parametrize("grid", GRIDS.values(), ids=GRIDS.keys())
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=DT_ID.get)
@pytest.mark.parametrize("path", [1, 2], ids=["valu", "mfma"])
@pytest.mark.parametrize("partition", [32, 64, 96, 512])
def test_decode_split_context(dtype, path, partition, grid):
    """Several partitions per sequence (equal sizes, rounded to 32 tokens),
    merged by the reduce kernel, with lengths around partition boundaries."""
    say("decode split", DT_ID[dtype], path, partition, grid)
    hq, hkv, hd, bs = 8, 2, 128, 16 if partition % 32 == 0 else 32
    lens = [1, partition - 1, partition, partition + 1, 3 * partition + 5, 1000, 17]
    q, kp, vp, tables, L = _case(300 + partition + path, lens, hq, hkv, hd, bs)
    _check_decode(q, kp, vp, tables, L, hkv, dtype, 1.0 / math.sqrt(hd),
                  partition=partition, path=path, grid=grid)


@pytest.mark.parametrize("path", [1, 2], ids=["valu", "mfma"])
def test_decode_split_context_any_workspace_contents(path):
    """The workspace needs no initialisation: one full of random bytes, used
    for several split calls in a row, gives the oracle's result every time."""
    say("decode split garbage workspace", path)
    hq, hkv, hd, bs = 8, 2, 128, 16
    lens = [1, 95, 96, 97, 1000, 333]
    q, kp, vp, tables, L = _case(350 + path, lens, hq, hkv, hd, bs)
    dev, (qt, kt, vt) = upload_case(q, kp, vp, tables, L, torch.bfloat16)
    want = oracle.decode(qt, kt, vt, tables, L, 0.1, hkv)
    need = pk.workspace_bytes(len(lens), hq, hkv, hd, bs, tables.shape[1], int(L.max()),
                              torch.bfloat16, 96, path)
    gen = torch.Generator(device=DEV).manual_seed(5)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device=DEV, generator=gen)
    for _ in range(3):
        out = torch.empty_like(dev["q"])
        pk.paged_attention_decode(out, dev["q"], dev["k"], dev["v"], dev["tables"], dev["lens"],
                                  0.1, int(L.max()), workspace=ws, partition_tokens=96, path=path)
        torch.cuda.synchronize()
        assert max_err(out, want) <= 2e-2


def test_decode_split_context_fp32():
    say("decode split fp32")
    lens = [1, 31, 32, 33, 500]
    q, kp, vp, tables, L = _case(400, lens, 4, 4, 64, 16)
    _check_decode(q, kp, vp, tables, L, 4, torch.float32, 0.125, partition=32)


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_ID.get)
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2)])
def test_decode_single_token_is_the_value_row(dtype, hq, hkv):
    say("decode L=1", DT_ID[dtype], hq, hkv)
    q, kp, vp, tables, L = _case(500, [1, 1, 1], hq, hkv, 128, 16)
    dev, (qt, kt, vt) = upload_case(q, kp, vp, tables, L, dtype)
    got = decode_gpu(dev["q"], dev["k"], dev["v"], dev["tables"], dev["lens"], 0.3).cpu()
    for s in range(3):
        b = int(tables[s, 0])
        for h in range(hq):
            assert torch.equal(got[s, h], vt[b, h // (hq // hkv), 0]), (s, h)


@pytest.mark.parametrize("path", [pk.PATH_VALU, pk.PATH_MFMA], ids=["valu", "mfma"])
def test_decode_zero_scale_is_the_mean_of_the_values(path):
    """scale = 0 weighs every token alike: the output is the mean of the
    sequence's V rows (split partitions included), with no NaN from the
    masked slots past the context."""
    say("decode scale 0", path)
    lens = [1, 19, 300, 700]
    q, kp, vp, tables, L = _case(501, lens, 8, 2, 128, 16)
    dev, (qt, kt, vt) = upload_case(q, kp, vp, tables, L, torch.bfloat16)
    got = decode_gpu(dev["q"], dev["k"], dev["v"], dev["tables"], dev["lens"], 0.0,
                     partition=256, path=path).cpu().double().numpy()
    assert np.isfinite(got).all()
    v = vt.double().numpy()
    for s, n in enumerate(lens):
        nb = -(-n // 16)
        rows = v[tables[s, :nb]].transpose(0, 2, 1, 3).reshape(nb * 16, 2, 128)[:n]
        mean = np.repeat(rows.mean(axis=0), 4, axis=0)
        assert np.abs(got[s] - mean).max() <= TOL[torch.bfloat16], s


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=DT_ID.get)
@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 2)])
def test_decode_placement_invariance_and_determinism(dtype, hq, hkv):
    """Moving the blocks (and rewriting the tables) and running again give
    bit-identical results: the arithmetic order depends only on logical
    positions, and nothing in the kernels is order-nondeterministic."""
    say("decode placement", DT_ID[dtype], hq, hkv)
    rng = np.random.default_rng(600)
    lens = [700, 33, 1200, 5]
    q, ks, vs, nblk = pins.random_case(rng, 4, hq, hkv, 128, lens, 16, extra_blocks=40)
    outs = []
    for rep in range(2):
        kp, vp, tables, L, _ = pins.page(ks, vs, 16, nblk, rng)
        dev, _ = upload_case(q, kp, vp, tables, L, dtype)
        for _ in range(2):
            outs.append(decode_gpu(dev["q"], dev["k"], dev["v"], dev["tables"], dev["lens"],
                                   0.088, partition=256).cpu())
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2)])
def test_decode_poisoned_slots_never_reach_the_result(hq, hkv):
    say("decode poison", hq, hkv)
    lens = [5, 17, 40, 129]
    r1 = _case(700, lens, hq, hkv, 128, 16, poison=True)
    r2 = _case(700, lens, hq, hkv, 128, 16, poison=False)
    g1, _ = _check_decode(*r1, hkv, torch.float16, 0.1, partition=64)
    g2, _ = _check_decode(*r2, hkv, torch.float16, 0.1, partition=64)
    assert torch.isfinite(g1).all()
    assert torch.equal(g1.view(torch.int16), g2.view(torch.int16))


@pytest.mark.parametrize("grid", GRIDS.values(), ids=GRIDS.keys())
@pytest.mark.parametrize("path", [1, 2], ids=["valu", "mfma"])
def test_decode_zero_length_gives_zeros(path, grid):
    say("decode L=0", path, grid)
    q, kp, vp, tables, L = _case(800, [0, 9, 0], 8, 2, 128, 16)
    dev, (qt, kt, vt) = upload_case(q, kp, vp, tables, L, torch.bfloat16)
    got = decode_gpu(dev["q"], dev["k"], dev["v"], dev["tables"], dev["lens"], 0.1, path=path,
                     grid=grid)
    assert not got[0].any() and not got[2].any()
    want = oracle.decode(qt, kt, vt, tables, L, 0.1, 2)
    assert max_err(got, want) <= 2e-2


@pytest.mark.parametrize("grid", GRIDS.values(), ids=GRIDS.keys())
@pytest.mark.parametrize("path", [1, 2], ids=["valu", "mfma"])
def test_decode_bad_table_entry_gives_nan_not_a_fault(path, grid):
    say("decode bad table", path, grid)
    q, kp, vp, tables, L = _case(900, [40, 40], 8, 2, 128, 16)
    tables = tables.copy()
    tables[1, 1] = kp.shape[0] + 1000          # outside the pool
    dev, (qt, kt, vt) = upload_case(q, kp, vp, tables, L, torch.float16)
    got = decode_gpu(dev["q"], dev["k"], dev["v"], dev["tables"], dev["lens"], 0.1, path=path,
                     grid=grid)
    assert torch.isnan(got[1]).all()
    want = oracle.decode(qt, kt, vt, tables, L, 0.1, 2, seqs=[0])
    assert max_err(got[:1], want[:1]) <= 2e-2


def test_decode_contiguous_control_matches_paged():
    """The contiguous-layout control reads block s*max_blocks + j; laid out
    that way it must equal the paged result bit for bit."""
    say("decode contiguous control")
    rng = np.random.default_rng(1000)
    lens = [100, 37, 256]
    hq, hkv, hd, bs = 8, 2, 128, 16
    q, ks, vs, _ = pins.random_case(rng, 3, hq, hkv, hd, lens, bs)
    maxb = 16
    kp = np.zeros((3 * maxb, hkv, bs, hd))
    vp = np.zeros((3 * maxb, hkv, bs, hd))
    tables = np.zeros((3, maxb), np.int64)
    for s, (k, v) in enumerate(zip(ks, vs)):
        nb = -(-len(k) // bs)
        tables[s, :nb] = s * maxb + np.arange(nb)
        for src, dst in ((k, kp), (v, vp)):
            pad = np.zeros((nb * bs, hkv, hd))
            pad[:len(src)] = src
            dst[s * maxb:s * maxb + nb] = pad.reshape(nb, bs, hkv, hd).transpose(0, 2, 1, 3)
    dev, (qt, kt, vt) = upload_case(q, kp, vp, tables, np.array(lens), torch.bfloat16)
    a = decode_gpu(dev["q"], dev["k"], dev["v"], dev["tables"], dev["lens"], 0.09)
    b = decode_gpu(dev["q"], dev["k"], dev["v"], None, dev["lens"], 0.09, max_len=256, path=3)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # and both against the oracle, which reads the same layout through the table
    want = oracle.decode(qt, kt, vt, tables, np.array(lens), 0.09, hkv)
    assert max_err(b, want) <= 2e-2


@pytest.mark.parametrize("hkv", [8, 2], ids=["mha-valu", "gqa-mfma"])
def test_decode_contiguous_control_against_oracle(hkv):
    """The no-table control on both kernels (MHA runs on the vector-ALU
    kernel, grouped heads on the MFMA one) against the float64 oracle given
    the identity tables s * W + j; fp16, ragged lengths."""
    say("decode contiguous control vs oracle", hkv)
    rng = np.random.default_rng(1001)
    lens = [1, 16, 17, 300, 511]
    hq, hd, bs = 8, 128, 16
    w = -(-max(lens) // bs)
    nb = len(lens) * w
    q = rng.standard_normal((len(lens), hq, hd))
    kp = rng.standard_normal((nb, hkv, bs, hd))
    vp = rng.standard_normal((nb, hkv, bs, hd))
    tables = (np.arange(len(lens))[:, None] * w + np.arange(w)[None, :]).astype(np.int64)
    dev, (qt, kt, vt) = upload_case(q, kp, vp, tables, np.array(lens), torch.float16)
    got = decode_gpu(dev["q"], dev["k"], dev["v"], None, dev["lens"], 0.088, max_len=max(lens),
                     path=3)
    want = oracle.decode(qt, kt, vt, tables, np.array(lens), 0.088, hkv)
    assert max_err(got, want) <= 2e-2


@pytest.mark.parametrize("grid", [0, 2], ids=["auto", "planned"])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=DT_ID.get)
@pytest.mark.parametrize("hq,hkv,partition", [(4, 4, 0), (8, 2, 0), (8, 2, 64), (2, 2, 32)])
def test_decode_many_sequences_longest_first(dtype, hq, hkv, partition, grid):
    """A large batch, longest first: ranked inside the direct grid's
    workgroups (auto, where the grid is large enough) or listed by the
    planner; lengths log-uniform so the order is far from the index order;
    partitions 64 and 32 run the split path under the order too."""
    say("decode longest first", DT_ID[dtype], hq, hkv, partition, grid)
    num_seqs, hd, bs = 800, 128, 16
    rng = np.random.default_rng(1100 + hq + partition)
    lens = np.clip(np.rint(np.exp(rng.uniform(0, math.log(300), num_seqs))), 1, 300).astype(int)
    q, ks, vs, nblk = pins.random_case(rng, num_seqs, hq, hkv, hd, lens, bs, extra_blocks=3)
    kp, vp, tables, L, _ = pins.page(ks, vs, bs, nblk, rng)
    from paged_kv_cache_389_amd import plan
    dt = {torch.float16: 1, torch.bfloat16: 2}[dtype]
    p = plan(num_seqs, hq, hkv, hd, bs, tables.shape[1], int(L.max()), dt, partition, 0, grid)
    if grid == 2 or hq == hkv:
        assert p["longest_first"], p
    _check_decode(q, kp, vp, tables, L, hkv, dtype, 1.0 / math.sqrt(hd), partition=partition,
                  grid=grid)


def test_decode_planned_batch_of_several_chunks():
    """More than 1024 sequences: the planner works in chunks of 1024, with
    empty sequences among them."""
    say("decode planned chunks")
    num_seqs, hq, hkv, hd, bs = 2500, 2, 2, 64, 16
    rng = np.random.default_rng(1200)
    lens = rng.integers(0, 97, num_seqs)
    lens[::37] = 0
    q, ks, vs, nblk = pins.random_case(rng, num_seqs, hq, hkv, hd, lens, bs, extra_blocks=3)
    kp, vp, tables, L, _ = pins.page(ks, vs, bs, nblk, rng)
    from paged_kv_cache_389_amd import GRID_PLANNED, plan
    assert plan(num_seqs, hq, hkv, hd, bs, tables.shape[1], int(L.max()), 1)["grid"] == \
        GRID_PLANNED
    got, _ = _check_decode(q, kp, vp, tables, L, hkv, torch.float16, 0.125, partition=32)
    assert not got[lens == 0].any()


@pytest.mark.parametrize("grid", GRIDS.values(), ids=GRIDS.keys())
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=DT_ID.get)
@pytest.mark.parametrize("hq,hkv", [(2, 2), (16, 2)])
def test_decode_long_sequence_many_partitions(dtype, hq, hkv, grid):
    """One long sequence cut into dozens of partitions among short and empty
    ones; the reduce merges dozens of partial states per head."""
    say("decode long many partitions", DT_ID[dtype], hq, hkv, grid)
    lens = [9000, 0, 3, 777, 0, 16]
    q, kp, vp, tables, L = _case(1300 + hq, lens, hq, hkv, 128, 16)
    got, _ = _check_decode(q, kp, vp, tables, L, hkv, dtype, 1.0 / math.sqrt(128), partition=256,
                           grid=grid)
    assert not got[1].any() and not got[4].any()


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 2)])
def test_decode_planned_determinism_and_placement(hq, hkv):
    """Planned grid: bit-identical results across runs and across physical
    placements of the same logical sequences."""
    say("decode planned placement", hq, hkv)
    rng = np.random.default_rng(1400)
    lens = [700, 33, 1200, 5, 2000, 1]
    q, ks, vs, nblk = pins.random_case(rng, len(lens), hq, hkv, 128, lens, 16, extra_blocks=40)
    outs = []
    for rep in range(2):
        kp, vp, tables, L, _ = pins.page(ks, vs, 16, nblk, rng)
        dev, _ = upload_case(q, kp, vp, tables, L, torch.float16)
        for _ in range(2):
            outs.append(decode_gpu(dev["q"], dev["k"], dev["v"], dev["tables"], dev["lens"],
                                   0.088, partition=256, grid=2).cpu())
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


def test_decode_largest_batch():
    """The largest batch the grid takes, 65,535 sequences (short and empty
    ones, as many single-block contexts): the planning kernel lists 64
    chunks of 1024; sampled sequences (every 997th, plus the longest) match
    the oracle and empty sequences give zero rows."""
    say("decode largest batch")
    num_seqs, hq, hkv, hd, bs = 65535, 2, 1, 64, 16
    rng = np.random.default_rng(1500)
    lens = rng.integers(0, 40, num_seqs)
    lens[::101] = 0
    nblk = -(-lens // bs)
    total = int(nblk.sum()) + 1
    perm = rng.permutation(total)
    width = int(nblk.max())
    tables = np.zeros((num_seqs, width), np.int32)
    starts = np.concatenate([[0], np.cumsum(nblk)[:-1]])
    for j in range(width):
        has = nblk > j
        tables[has, j] = perm[starts[has] + j]
    q = rng.standard_normal((num_seqs, hq, hd)).astype(np.float16)
    kp = rng.standard_normal((total, hkv, bs, hd)).astype(np.float16)
    vp = rng.standard_normal((total, hkv, bs, hd)).astype(np.float16)
    got = decode_gpu(torch.from_numpy(q).to(DEV), torch.from_numpy(kp).to(DEV),
                     torch.from_numpy(vp).to(DEV), torch.from_numpy(tables).to(DEV),
                     torch.from_numpy(lens.astype(np.int32)).to(DEV), 0.125)
    g = got.cpu().double().numpy()
    assert np.isfinite(g).all()
    assert not g[lens == 0].any()
    seqs = sorted(set(range(0, num_seqs, 997)) | {int(np.argmax(lens))})
    want = oracle.decode(q, kp, vp, tables, lens, 0.125, hkv, seqs=seqs)
    assert float(np.abs(g[seqs] - want[seqs]).max()) <= TOL[torch.float16]


@pytest.mark.parametrize("dtype,hq,hkv", [(torch.float16, 8, 8), (torch.bfloat16, 8, 2),
                                          (torch.float32, 4, 4)], ids=["mha", "gqa", "fp32"])
def test_shared_blocks_flag_changes_only_the_load_policy(dtype, hq, hkv):
    """Forks of one prompt (shared blocks): the decode with
    PKV_PATH_SHARED_BLOCKS (cached K/V loads) and without it (streaming
    loads) give bit-identical rows, which match the oracle; also on a split
    and on the planned grid."""
    from paged_kv_cache_389_amd import workloads
    say("shared-blocks flag", DT_ID[dtype], hq, hkv)
    wl = workloads.build_sharing(dtype={torch.float16: "fp16", torch.bfloat16: "bf16",
                                        torch.float32: "fp32"}[dtype],
                                 num_prompts=3, fanout=5, prompt_len=300, max_gen=40,
                                 num_heads=hq, head_dim=128, block_size=16, num_blocks=512,
                                 device=DEV)
    if hkv != hq:   # grouped heads: keep the first hkv KV heads of the pools
        wl.k_cache = wl.k_cache[:, :hkv].contiguous()
        wl.v_cache = wl.v_cache[:, :hkv].contiguous()
        wl.num_kv_heads = hkv
    tables = torch.from_numpy(wl.block_tables).to(DEV)
    lens = torch.from_numpy(wl.context_lens).to(DEV)
    want = oracle.decode(wl.q.cpu(), wl.k_cache.cpu(), wl.v_cache.cpu(), wl.block_tables,
                         wl.context_lens, wl.scale, hkv)
    for partition, grid in ((0, 0), (64, 1), (64, 2)):
        a = decode_gpu(wl.q, wl.k_cache, wl.v_cache, tables, lens, wl.scale,
                       partition=partition, grid=grid)
        b = decode_gpu(wl.q, wl.k_cache, wl.v_cache, tables, lens, wl.scale,
                       partition=partition, grid=grid, path=pk.PATH_SHARED_BLOCKS)
        assert torch.equal(a.view(INT_VIEW[dtype]), b.view(INT_VIEW[dtype]))
        assert max_err(b, want) <= TOL[dtype]
