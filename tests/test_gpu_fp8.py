"""The 8-bit (OCP E4M3) KV cache on the GPU, against the oracle:

* the quantising cache write, byte for byte over the whole cache, for
  float32, float16 and bfloat16 sources, with the format's edge values
  (ties, saturation, subnormals, signed zeros, infinities, NaN) and the
  float32-quotient cases of the hand-worked fixture;
* every one of the 256 codes read back through V (exact) and through K
  (one-hot queries), which pins the device's code conversions;
* decode over random code caches for every query type, MHA and grouped
  heads, both kernels (vector ALU and MFMA), several head and block sizes,
  both grids and forced splits, within 1e-5 (float32 queries) or 2e-2
  (16-bit);
* a quantise-then-attend round trip through the block manager's slots."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8
from gpu_helpers import DEV, TOL, say
from paged_kv_cache_389_amd import _native as pk

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.float16, torch.bfloat16]
DT_ID = {torch.float32: "fp32", torch.float16: "fp16", torch.bfloat16: "bf16"}
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")


def _edge_values(k_scale):
    """float32 sources whose quotients by k_scale hit the format's edges."""
    mags = fp8.e4m3_value(np.arange(0, 0x7F))
    mids = (mags[1:] + mags[:-1]) / 2
    q = np.concatenate([mags, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e4),
                        [448.0, 449.0, 464.0, 480.0, 1e6, np.inf, 2.0 ** -10, 2.0 ** -12,
                         0.0, np.nan]])
    q = np.concatenate([q, -q])
    return (q * k_scale).astype(np.float32)


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_ID.get)
def test_reshape_and_cache_fp8_bit_exact(dtype):
    say("reshape_and_cache_fp8", DT_ID[dtype])
    g = torch.Generator().manual_seed(301)
    nb, hkv, bs, hd, ntok = 24, 2, 16, 128, 40
    k_scale, v_scale = 0.25, 0.0390625
    k = (torch.randn((ntok, hkv, hd), generator=g) * 3).to(dtype)
    v = (torch.randn((ntok, hkv, hd), generator=g) * 3).to(dtype)
    if dtype == torch.float32:
        edges = torch.from_numpy(_edge_values(k_scale))
        flat = k.view(-1)
        flat[:edges.numel()] = edges
        fx = json.load(open(os.path.join(GOLDEN, "fp8_e4m3_quantise.json")))
        # the fixture's float32-quotient cases, written as V sources under their scale
        c = fx["float32_quotient_cases"][0]
        v_scale = c["scale"]
        v.view(-1)[:2] = torch.tensor([c["x"], -c["x"]], dtype=torch.float32)
    else:
        k.view(-1)[:4] = torch.tensor([float("inf"), float("-inf"), float("nan"), -0.0]).to(dtype)
    slots = torch.randperm(nb * bs, generator=g)[:ntok].to(torch.int64)
    slots[3] = -1                      # skipped
    slots[7] = nb * bs + 5             # past the pool: skipped
    kc0 = torch.randint(0, 256, (nb, hkv, bs, hd), generator=g, dtype=torch.uint8)
    vc0 = torch.randint(0, 256, (nb, hkv, bs, hd), generator=g, dtype=torch.uint8)
    kc, vc = kc0.to(DEV), vc0.to(DEV)
    pk.reshape_and_cache_fp8(k.to(DEV), v.to(DEV), kc, vc, slots.to(DEV), k_scale, v_scale)
    torch.cuda.synchronize()
    want_k, want_v = kc0.numpy().copy(), vc0.numpy().copy()
    ok_slots = np.where(slots.numpy() < nb * bs, slots.numpy(), -1)
    fp8.reshape_and_cache_fp8(k, v, want_k, want_v, ok_slots, k_scale, v_scale)
    got_k, got_v = kc.cpu().numpy(), vc.cpu().numpy()
    bad = np.argwhere(got_k != want_k)
    assert bad.size == 0, f"{len(bad)} K codes differ, first {bad[:3].tolist()}: " \
        f"{got_k[tuple(bad[0])]:#x} vs {want_k[tuple(bad[0])]:#x}"
    assert np.array_equal(got_v, want_v)
    if dtype == torch.float32:
        b, o = divmod(int(slots[0]), bs)
        assert got_v[b, 0, o, :2].tolist() == [0x6A, 0xEA]


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_ID.get)
def test_every_code_reads_back(dtype):
    """V: two one-token sequences whose V rows hold codes 0..127 and
    128..255; the output is value(code) * v_scale exactly (NaN for the NaN
    codes).  K: 256 one-hot queries, each against a key row holding one code
    at its dimension, beside a zero key and one-hot values, so the output is
    sigmoid(value(code) * k_scale * scale)."""
    say("fp8 code read-back", DT_ID[dtype])
    hd, bs = 128, 16
    # V read-back
    vc = np.zeros((2, 1, bs, hd), np.uint8)
    vc[0, 0, 0] = np.arange(128)
    vc[1, 0, 0] = np.arange(128, 256)
    q = torch.zeros((2, 1, hd), dtype=dtype)
    tables = np.array([[0], [1]], np.int32)
    lens = np.array([1, 1], np.int32)
    out = torch.empty((2, 1, hd), dtype=dtype, device=DEV)
    zero_k = torch.zeros((2, 1, bs, hd), dtype=torch.uint8, device=DEV)   # finite scores
    pk.paged_attention_decode_fp8(out, q.to(DEV), zero_k, torch.from_numpy(vc).to(DEV),
                                  torch.from_numpy(tables).to(DEV),
                                  torch.from_numpy(lens).to(DEV), 1.0, 1.0, 0.5, 1)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy().reshape(-1)
    want = fp8.e4m3_value(np.arange(256)) * 0.5
    want = torch.from_numpy(want).to(dtype).double().numpy()   # rounding to the output type
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])

    # K read-back: sequence s, head h probes code p = 8 s + h at dim p % 128
    B, H = 32, 8
    kc = np.zeros((2 * B, H, bs, hd), np.uint8)
    vcb = np.zeros((2 * B, H, bs, hd), np.uint8)
    qk = np.zeros((B, H, hd), np.float32)
    for s in range(B):
        for h in range(H):
            p = 8 * s + h
            kc[2 * s, h, 0, p % hd] = p          # token 0: the probed code
            vcb[2 * s, h, 0, :] = 0x38           # token 0's value row: 1.0
            qk[s, h, p % hd] = 1.0               # token 1 (slot 1): zero key, zero value
    tables = np.stack([np.arange(0, 2 * B, 2)], 1).astype(np.int32)
    lens = np.full(B, 2, np.int32)
    k_scale, scale = 1.0 / 64, 0.125
    qd = torch.from_numpy(qk).to(dtype)
    out = torch.empty((B, H, hd), dtype=dtype, device=DEV)
    pk.paged_attention_decode_fp8(out, qd.to(DEV), torch.from_numpy(kc).to(DEV),
                                  torch.from_numpy(vcb).to(DEV), torch.from_numpy(tables).to(DEV),
                                  torch.from_numpy(lens).to(DEV), scale, k_scale, 1.0, 2)
    torch.cuda.synchronize()
    want = fp8.decode_fp8(qd, kc, vcb, tables, lens, scale, k_scale, 1.0, H)
    got = out.cpu().double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    err = float(np.abs(got[ok] - want[ok]).max())
    assert err <= TOL[dtype], err
    # every finite code gives its own weight: the probes are distinct
    w = np.array([got[s, h, 0] for s in range(B) for h in range(H)])   # probe p = 8 s + h
    assert np.isnan(w[0x7F]) and np.isnan(w[0xFF])


CASES = [
    # dtype, hq, hkv, hd, bs, grid, partition, path (0 auto: MFMA for 16-bit grouped heads)
    (torch.float32, 4, 4, 64, 16, 0, 0, 0),
    (torch.float16, 8, 8, 128, 16, 0, 0, 0),
    (torch.bfloat16, 8, 2, 128, 16, 0, 0, 0),
    (torch.bfloat16, 8, 2, 128, 16, 0, 0, 1),
    (torch.float16, 16, 4, 128, 32, 2, 0, 0),
    (torch.float16, 64, 8, 128, 32, 1, 128, 2),
    (torch.bfloat16, 12, 3, 64, 16, 2, 64, 2),
    (torch.bfloat16, 8, 8, 256, 8, 1, 64, 0),
    (torch.float16, 8, 1, 128, 8, 2, 96, 0),
    (torch.float32, 4, 2, 128, 32, 1, 128, 0),
]


@pytest.mark.parametrize("dtype,hq,hkv,hd,bs,grid,partition,path", CASES,
                         ids=lambda v: DT_ID.get(v, str(v)))
def test_decode_fp8_matches_oracle(dtype, hq, hkv, hd, bs, grid, partition, path):
    say("decode_fp8", DT_ID[dtype], hq, hkv, hd, bs, grid, partition, path)
    rng = np.random.default_rng(hq * 1000 + hd + bs + grid)
    B = 9
    lens = np.array([1, 2, bs, bs + 1, 3 * bs - 1, 7 * bs + 3, 200, 517, 0], np.int32)[:B]
    nblk = -(-lens // bs)
    nb = int(nblk.sum()) + 5
    perm = rng.permutation(nb)
    tables = np.zeros((B, int(nblk.max())), np.int32)
    at = 0
    for s in range(B):
        tables[s, :nblk[s]] = perm[at:at + nblk[s]]
        at += nblk[s]
    kc = rng.integers(0, 256, (nb, hkv, bs, hd)).astype(np.uint8)
    vc = rng.integers(0, 256, (nb, hkv, bs, hd)).astype(np.uint8)
    for c in (kc, vc):
        c[(c & 0x7F) == 0x7F] = 0x00
    # NaN in every slot no sequence reads: masking must keep them out
    used = np.zeros((nb, bs), bool)
    for s in range(B):
        for t in range(lens[s]):
            used[tables[s, t // bs], t % bs] = True
    for b in range(nb):
        for o in range(bs):
            if not used[b, o]:
                kc[b, :, o, :] = 0x7F
                vc[b, :, o, :] = 0xFF
    q = torch.randn((B, hq, hd), generator=torch.Generator().manual_seed(5)).to(dtype)
    # uniform codes reach 448: these scales keep |k| <= 4.7 and |v| <= 3.5, so
    # rounding the output to a 16-bit type stays inside the tolerance
    k_scale, v_scale, scale = 1.0 / 96, 1.0 / 128, 1.0 / math.sqrt(hd)
    out = torch.empty((B, hq, hd), dtype=dtype, device=DEV)
    pk.paged_attention_decode_fp8(out, q.to(DEV), torch.from_numpy(kc).to(DEV),
                                  torch.from_numpy(vc).to(DEV), torch.from_numpy(tables).to(DEV),
                                  torch.from_numpy(lens).to(DEV), scale, k_scale, v_scale,
                                  int(lens.max()), partition_tokens=partition, grid=grid,
                                  path=path)
    torch.cuda.synchronize()
    want = fp8.decode_fp8(q, kc, vc, tables, lens, scale, k_scale, v_scale, hkv)
    got = out.cpu().double().numpy()
    assert np.isfinite(got).all()
    err = float(np.abs(got - want).max())
    assert err <= TOL[dtype], f"max abs err {err}"


def test_quantise_then_attend_round_trip():
    """New tokens quantised into slots by the device, then attended to: the
    result matches the oracle's quantise-then-attend on the same sources."""
    say("fp8 quantise then attend")
    from paged_kv_cache_389_amd.block_manager import BlockManager
    rng = np.random.default_rng(17)
    hq, hkv, hd, bs, nb = 16, 4, 128, 16, 96
    bm = BlockManager(nb, bs, free_order=rng.permutation(nb))
    seqs = [bm.new_sequence() for _ in range(5)]
    lens = [1, 16, 33, 250, 97]
    slots = np.concatenate([bm.extend(s, L) for s, L in zip(seqs, lens)])
    k = torch.randn((len(slots), hkv, hd), generator=torch.Generator().manual_seed(3))
    v = torch.randn((len(slots), hkv, hd), generator=torch.Generator().manual_seed(4))
    k, v = k.to(torch.bfloat16), v.to(torch.bfloat16)
    k_scale = float(k.abs().max()) / 448
    v_scale = float(v.abs().max()) / 448
    kc = torch.zeros((nb, hkv, bs, hd), dtype=torch.uint8, device=DEV)
    vc = torch.zeros_like(kc)
    pk.reshape_and_cache_fp8(k.to(DEV), v.to(DEV), kc, vc, torch.from_numpy(slots).to(DEV),
                             k_scale, v_scale)
    tables = bm.block_table_array(seqs)
    cl = bm.context_lens(seqs)
    q = torch.randn((5, hq, hd), generator=torch.Generator().manual_seed(6)).to(torch.bfloat16)
    out = torch.empty((5, hq, hd), dtype=torch.bfloat16, device=DEV)
    pk.paged_attention_decode_fp8(out, q.to(DEV), kc, vc, torch.from_numpy(tables).to(DEV),
                                  torch.from_numpy(cl).to(DEV), 1 / math.sqrt(hd), k_scale,
                                  v_scale, int(cl.max()))
    torch.cuda.synchronize()
    kw = np.zeros((nb, hkv, bs, hd), np.uint8)
    vw = np.zeros_like(kw)
    fp8.reshape_and_cache_fp8(k, v, kw, vw, slots, k_scale, v_scale)
    assert np.array_equal(kc.cpu().numpy(), kw) and np.array_equal(vc.cpu().numpy(), vw)
    want = fp8.decode_fp8(q, kw, vw, tables, cl, 1 / math.sqrt(hd), k_scale, v_scale, hkv)
    err = float(np.abs(out.cpu().double().numpy() - want).max())
    assert err <= TOL[torch.bfloat16], err
    # and the quantisation error against unquantised attention stays within
    # half a code step at the largest values (3 fraction bits: amax / 16)
    exact = oracle.decode(q, k_pool(k, slots, nb, bs), k_pool(v, slots, nb, bs), tables, cl,
                          1 / math.sqrt(hd), hkv)
    assert float(np.abs(want - exact).max()) < float(v.abs().max()) / 16


def k_pool(rows, slots, nb, bs):
    pool = np.zeros((nb, rows.shape[1], bs, rows.shape[2]))
    r = rows.double().numpy()
    for j, s in enumerate(slots):
        pool[s // bs, :, s % bs, :] = r[j]
    return pool


FULL = {"opt13b_fp16": (6, 512), "llama3_8b_gqa_bf16": (6, 1024),
        "long_context_gqa_bf16": (2, 1024)}


def _oracle_codes_16bit(pool, scale):
    """The oracle's codes of every element of a 16-bit device pool.  A code
    depends only on the element's value and the scale, and a 16-bit element
    has 65,536 bit patterns, so the oracle quantises each pattern once and
    every element takes its pattern's code (the oracle applied to every
    element, without encoding the same value twice)."""
    patterns = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(pool.dtype)
    table = fp8.quantize(patterns, scale)
    bits = pool.view(torch.int16).cpu().numpy().view(np.uint16)
    return table[bits]


def test_oracle_codes_by_pattern_equal_direct_quantisation():
    """The per-pattern shortcut of the full-size check equals the oracle
    applied element by element (NaN, infinities and both zeros included)."""
    g = torch.Generator().manual_seed(7)
    x = (torch.randn(4000, generator=g) * 300).to(torch.bfloat16)
    x[:4] = torch.tensor([float("nan"), float("inf"), -0.0, 0.0], dtype=torch.bfloat16)
    for sc in (0.37, 1.0, 2.5e-3):
        assert np.array_equal(_oracle_codes_16bit(x, sc), fp8.quantize(x, sc))


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_fp8_matches_oracle(name):
    """The workloads at full size with 8-bit pools: the library quantises
    every slot (both whole code buffers compared with the oracle's codes), then
    decode_fp8 runs in the library's own configuration and with a forced
    split on the planned grid; sampled sequences (the longest, the shortest,
    seeded others; all heads) are compared with the oracle."""
    from paged_kv_cache_389_amd import workloads
    from gpu_helpers import compact_pool
    n_sample, split = FULL[name]
    say("full-size fp8 build", name)
    wl = workloads.make(name, device=DEV)
    nb, hkv, bs, hd = wl.k_cache.shape
    k_scale = float(wl.k_cache.abs().amax().float()) / 448
    v_scale = float(wl.v_cache.abs().amax().float()) / 448
    kc = torch.empty((nb, hkv, bs, hd), dtype=torch.uint8, device=DEV)
    vc = torch.empty_like(kc)
    chunk = 1024
    for b0 in range(0, nb, chunk):
        b1 = min(nb, b0 + chunk)
        rk = wl.k_cache[b0:b1].permute(0, 2, 1, 3).reshape(-1, hkv, hd).contiguous()
        rv = wl.v_cache[b0:b1].permute(0, 2, 1, 3).reshape(-1, hkv, hd).contiguous()
        pk.reshape_and_cache_fp8(rk, rv, kc, vc,
                                 torch.arange(b0 * bs, b1 * bs, dtype=torch.int64, device=DEV),
                                 k_scale, v_scale)
    torch.cuda.synchronize()
    # the whole K and V code buffers against the oracle's codes of every slot
    say("full-size fp8 whole-buffer codes", name)
    for src, codes, sc in ((wl.k_cache, kc, k_scale), (wl.v_cache, vc, v_scale)):
        want_codes = _oracle_codes_16bit(src, sc)
        assert np.array_equal(codes.cpu().numpy(), want_codes), "quantised pool differs"
        del want_codes
    rng = np.random.default_rng(wl.seed)

    L = wl.context_lens
    seqs = [int(np.argmax(L)), int(np.argmin(L))]
    for s in rng.permutation(wl.num_seqs).tolist():
        if len(seqs) >= n_sample:
            break
        if s not in seqs:
            seqs.append(s)
    seqs = sorted(seqs)
    # the sampled sequences' blocks, compacted, as codes for the oracle
    wl_codes = workloads.Workload(**{**wl.__dict__, "k_cache": kc, "v_cache": vc})
    kcs, vcs, tables = compact_pool(wl_codes, seqs)
    want = fp8.decode_fp8(wl.q.cpu(), kcs.numpy(), vcs.numpy(), tables, L, wl.scale, k_scale,
                          v_scale, wl.num_kv_heads, seqs=seqs)
    tab = torch.from_numpy(wl.block_tables).to(DEV)
    lens = torch.from_numpy(L).to(DEV)
    for partition, grid in ((0, pk.GRID_AUTO), (split, pk.GRID_PLANNED)):
        say("full-size fp8 decode", name, partition, grid)
        out = torch.empty_like(wl.q)
        pk.paged_attention_decode_fp8(out, wl.q, kc, vc, tab, lens, wl.scale, k_scale, v_scale,
                                      wl.max_context_len, partition_tokens=partition, grid=grid)
        torch.cuda.synchronize()
        got = out.cpu().double().numpy()[seqs]
        assert np.isfinite(got).all()
        err = float(np.abs(got - want[seqs]).max())
        assert err <= TOL[wl.dtype], f"{name} partition {partition}: max abs err {err}"


def test_copy_and_swap_move_code_blocks_bit_exact():
    """copy_blocks and swap_blocks on uint8 code pools (dtype PKV_E4M3):
    whole blocks, byte for byte, against the oracle."""
    say("fp8 copy/swap")
    g = torch.Generator().manual_seed(401)
    nb, nh, hkv, bs, hd = 40, 12, 4, 16, 128
    kc0 = torch.randint(0, 256, (nb, hkv, bs, hd), generator=g, dtype=torch.uint8)
    vc0 = torch.randint(0, 256, (nb, hkv, bs, hd), generator=g, dtype=torch.uint8)
    kc, vc = kc0.to(DEV), vc0.to(DEV)
    pairs = np.array([[3, 30], [7, 31], [39, 0], [5, 99]], np.int64)
    pk.copy_blocks(kc, vc, torch.from_numpy(pairs).to(DEV))
    want_k, want_v = kc0.numpy().copy(), vc0.numpy().copy()
    oracle.copy_blocks(want_k, want_v, pairs[:3])
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), want_k) and np.array_equal(vc.cpu().numpy(), want_v)
    hk = torch.zeros((nh, hkv, bs, hd), dtype=torch.uint8).pin_memory()
    hv = torch.zeros((nh, hkv, bs, hd), dtype=torch.uint8).pin_memory()
    out_pairs = np.array([[30, 2], [1, 11], [17, 0]], np.int64)
    pk.swap_blocks(kc, vc, hk, hv, torch.from_numpy(out_pairs).to(DEV))
    torch.cuda.synchronize()
    hk_want = np.zeros((nh, hkv, bs, hd), np.uint8)
    hv_want = np.zeros_like(hk_want)
    oracle.swap_blocks(want_k, want_v, hk_want, hv_want, out_pairs)
    assert np.array_equal(hk.numpy(), hk_want) and np.array_equal(hv.numpy(), hv_want)
