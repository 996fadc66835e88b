"""Grouped decode on the GPU against the float64 oracle.

pkv_paged_attention_decode_grouped reads each tile that several sequences
share once for all of them; every output row must still be the plain decode
attention of its sequence.  Cases: forked prompts (parallel sampling) and
beam search, with multi-head and grouped-query heads, head dims 64 and 128,
block sizes 16 and 32, every slot no sequence owns poisoned with NaN;
groups of unrelated sequences (nothing shared: the result must not depend on
the grouping); empty and one-token contexts; the full-size sharing and beam
workloads on sampled rows; an out-of-pool block (NaN rows, no fault); and
PKV_DEBUG=1 rejecting malformed tile lists.  Bar: max-abs 2e-2 against the
unrounded oracle (16-bit inputs, fp32 accumulation)."""

import numpy as np
import pytest
import torch

import oracle
import pins
from gpu_helpers import DEV, TOL, decode_gpu, max_err, oracle_sample, say, upload_case
from paged_kv_cache_389_amd import _native as pk
from paged_kv_cache_389_amd import block_manager as bmod
from paged_kv_cache_389_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")


def _lists(tables, lens, groups, bs, max_members):
    members, tiles, start = bmod.group_tiles(tables, lens, groups, bs, max_members)
    if tiles.shape[0] == 0:
        tiles = np.zeros((1, 4), np.int32)
    return (torch.from_numpy(members).to(DEV), torch.from_numpy(tiles).to(DEV),
            torch.from_numpy(start).to(DEV), int(np.diff(start).max(initial=0)))


def _grouped(q, kc, vc, lens_d, lists, scale, max_len, part_tiles=0):
    members, tiles, start, max_group_tiles = lists
    out = torch.full_like(q, float("nan"))
    pk.paged_attention_decode_grouped(out, q, kc, vc, lens_d, members, tiles, start, scale,
                                      max_len, part_tiles=part_tiles,
                                      max_group_tiles=max_group_tiles)
    torch.cuda.synchronize()
    return out


PARTS = [0, 3, 16]   # whole groups, and parts of 3 / 16 tiles merged by the second kernel


def _poison_unowned(kc, vc, tables, lens, bs):
    """NaN in every slot that no sequence's first L tokens occupy."""
    owned = torch.zeros(kc.shape[0], bs, dtype=torch.bool)
    for s in range(len(lens)):
        for t in range(int(lens[s])):
            owned[int(tables[s][t // bs]), t % bs] = True
    mask = (~owned).to(DEV)[:, None, :, None].expand_as(kc)
    kc.masked_fill_(mask, float("nan"))
    vc.masked_fill_(mask, float("nan"))


def _check(wl, max_members, part_tiles=0, q=None):
    q = wl.q if q is None else q
    kc, vc = wl.k_cache, wl.v_cache
    _poison_unowned(kc, vc, wl.block_tables, wl.context_lens, wl.block_size)
    groups = bmod.share_groups(wl.block_tables, wl.context_lens, max_members)
    lists = _lists(wl.block_tables, wl.context_lens, groups, wl.block_size, max_members)
    lens_d = torch.from_numpy(wl.context_lens).to(DEV)
    got = _grouped(q, kc, vc, lens_d, lists, wl.scale, int(wl.context_lens.max()), part_tiles)
    want = oracle.decode(q.cpu(), kc.cpu(), vc.cpu(), wl.block_tables, wl.context_lens,
                         wl.scale, wl.num_kv_heads)
    err = max_err(got, want)
    assert err <= TOL[q.dtype], f"max abs err {err}"
    # the plain decode of the same batch agrees too (same bar against the oracle)
    plain = decode_gpu(q, kc, vc, torch.from_numpy(wl.block_tables).to(DEV), lens_d, wl.scale)
    assert max_err(plain, want) <= TOL[q.dtype]
    return groups


@pytest.mark.parametrize("part_tiles", PARTS)
@pytest.mark.parametrize("dtype,hd,bs,heads,fanout", [
    (torch.float16, 128, 16, 8, 8),
    (torch.bfloat16, 64, 32, 4, 16),
    (torch.bfloat16, 128, 32, 2, 8),
    (torch.float16, 64, 16, 3, 5),
])
def test_forked_prompts(dtype, hd, bs, heads, fanout, part_tiles):
    say("grouped forked prompts", dtype, hd, bs, heads, fanout, part_tiles)
    wl = workloads.build_sharing(dtype=dtype, num_prompts=5, fanout=fanout, prompt_len=70,
                                 prompt_extra=(1, 15), max_gen=40, num_heads=heads,
                                 head_dim=hd, block_size=bs, num_blocks=512,
                                 seed=300 + hd + bs + fanout, device=DEV)
    groups = _check(wl, fanout, part_tiles)
    assert max(len(g) for g in groups) == fanout   # the forks did share


@pytest.mark.parametrize("part_tiles", PARTS)
@pytest.mark.parametrize("dtype,hq,hkv,hd,bs,width", [
    (torch.bfloat16, 16, 4, 128, 16, 4),    # G = 4: 4 beams x 4 heads = 16 columns
    (torch.float16, 8, 4, 128, 32, 8),      # G = 2
    (torch.float16, 24, 8, 64, 16, 5),      # G = 3: 15 columns used
    (torch.bfloat16, 8, 8, 128, 16, 8),     # multi-head
])
def test_beam_search_batch(dtype, hq, hkv, hd, bs, width, part_tiles):
    say("grouped beam search", dtype, hq, hkv, hd, bs, width, part_tiles)
    wl = workloads.build_beam_search(dtype=dtype, num_requests=5, beam_width=width,
                                     prompt_lens=(3, 90), steps=30, num_q_heads=hq,
                                     num_kv_heads=hkv, head_dim=hd, block_size=bs,
                                     num_blocks=512, seed=400 + hq + bs, device=DEV)
    _check(wl, width, part_tiles)


@pytest.mark.parametrize("part_tiles", [0, 2])
@pytest.mark.parametrize("max_members", [1, 3, 16])
def test_unrelated_sequences_any_grouping(max_members, part_tiles):
    """Nothing shared: each tile has one member, and grouping must not change
    any row (empty and one-token contexts included)."""
    say("grouped unrelated", max_members)
    rng = np.random.default_rng(17 + max_members)
    lens = np.array([0, 1, 15, 16, 17, 130, 3, 64, 250, 33, 1, 200], dtype=np.int64)
    hq = hkv = 1
    q, ks, vs, nblk = pins.random_case(rng, len(lens), hq, hkv, 128, lens, 16, 4)
    kp, vp, tables, L, _ = pins.page(ks, vs, 16, nblk, rng, poison=True)
    dev, (qt, kt, vt) = upload_case(q, kp, vp, tables, L, torch.float16)
    order = rng.permutation(len(lens))
    groups = [list(map(int, order[i:i + max_members])) for i in range(0, len(order), max_members)]
    lists = _lists(tables, L, groups, 16, max_members)
    got = _grouped(dev["q"], dev["k"], dev["v"], dev["lens"], lists, 0.09, int(L.max()),
                   part_tiles)
    want = oracle.decode(qt, kt, vt, tables, L, 0.09, hkv)
    assert max_err(got, want) <= TOL[torch.float16]
    assert torch.all(got[0] == 0)   # the empty context: zero row


def test_sequences_outside_groups_are_not_written():
    say("grouped partial batch")
    rng = np.random.default_rng(5)
    lens = np.array([20, 40, 60, 80], dtype=np.int64)
    q, ks, vs, nblk = pins.random_case(rng, 4, 2, 2, 64, lens, 16, 2)
    kp, vp, tables, L, _ = pins.page(ks, vs, 16, nblk, rng, poison=True)
    dev, (qt, kt, vt) = upload_case(q, kp, vp, tables, L, torch.bfloat16)
    lists = _lists(tables, L, [[2, 0]], 16, 2)
    got = _grouped(dev["q"], dev["k"], dev["v"], dev["lens"], lists, 0.125, 80)
    want = oracle.decode(qt, kt, vt, tables, L, 0.125, 2)
    assert max_err(got[[0, 2]], want[[0, 2]]) <= TOL[torch.bfloat16]
    assert torch.isnan(got[[1, 3]]).all()   # left as the caller filled them


@pytest.mark.parametrize("part_tiles", [0, 2])
def test_out_of_pool_block_gives_nan_rows(part_tiles):
    say("grouped bad block")
    wl = workloads.build_sharing(dtype=torch.float16, num_prompts=3, fanout=4, prompt_len=40,
                                 max_gen=20, num_heads=2, head_dim=128, num_blocks=128,
                                 seed=9, device=DEV)
    groups = bmod.share_groups(wl.block_tables, wl.context_lens, 4)
    members, tiles, start = bmod.group_tiles(wl.block_tables, wl.context_lens, groups,
                                             wl.block_size, 4)
    tiles[int(start[1]) + 2, 0] = wl.num_blocks + 7   # a tile of group 1 outside the pool
    lists = (torch.from_numpy(members).to(DEV), torch.from_numpy(tiles).to(DEV),
             torch.from_numpy(start).to(DEV), int(np.diff(start).max()))
    lens_d = torch.from_numpy(wl.context_lens).to(DEV)
    got = _grouped(wl.q, wl.k_cache, wl.v_cache, lens_d, lists, wl.scale,
                   int(wl.context_lens.max()), part_tiles)
    want = oracle.decode(wl.q.cpu(), wl.k_cache.cpu(), wl.v_cache.cpu(), wl.block_tables,
                         wl.context_lens, wl.scale, wl.num_kv_heads)
    bad = [s for s in groups[1]]
    good = [s for g in (groups[0], groups[2]) for s in g]
    assert torch.isnan(got[bad]).all()
    assert max_err(got[good], want[good]) <= TOL[torch.float16]


@pytest.mark.parametrize("part_tiles", [0, 32])
@pytest.mark.parametrize("name", ["sharing_fp16", "beam_search_fp16", "system_prompt_bf16"])
def test_full_size_workloads_sampled(name, part_tiles):
    """The grouped decode at full size: forks of one prompt, beams, and
    distinct requests sharing cached system prompts (grouped heads: 16 / G
    members per group), against the oracle on sampled rows and against the
    per-sequence decode."""
    say("grouped full size", name, part_tiles)
    wl = workloads.make(name, device=DEV)
    mm = min(8, 16 // wl.group)
    groups = bmod.share_groups(wl.block_tables, wl.context_lens, mm)
    if name == "system_prompt_bf16":
        assert all(len(g) == mm for g in groups)   # every group shares a prompt
    lists = _lists(wl.block_tables, wl.context_lens, groups, wl.block_size, mm)
    lens_d = torch.from_numpy(wl.context_lens).to(DEV)
    got = _grouped(wl.q, wl.k_cache, wl.v_cache, lens_d, lists, wl.scale,
                   int(wl.context_lens.max()), part_tiles)
    rng = np.random.default_rng(1)
    seqs = sorted(set(int(s) for s in rng.choice(wl.num_seqs, 12, replace=False)) |
                  {int(np.argmax(wl.context_lens)), int(np.argmin(wl.context_lens))})
    heads = [0, wl.num_q_heads // 2, wl.num_q_heads - 1]
    want = oracle_sample(wl, seqs, heads)
    g = got.cpu().double().numpy()
    err = max(float(np.abs(g[s, h] - want[s, h]).max()) for s in seqs for h in heads)
    assert err <= TOL[wl.dtype], f"max abs err {err}"
    plain = decode_gpu(wl.q, wl.k_cache, wl.v_cache, torch.from_numpy(wl.block_tables).to(DEV),
                       lens_d, wl.scale)
    assert float((plain.float() - got.float()).abs().max()) <= 2 * TOL[wl.dtype]


def test_debug_rejects_bad_lists(monkeypatch):
    say("grouped debug checks")
    monkeypatch.setenv("PKV_DEBUG", "1")
    wl = workloads.build_sharing(dtype=torch.float16, num_prompts=2, fanout=3, prompt_len=40,
                                 max_gen=10, num_heads=2, head_dim=64, num_blocks=64, seed=3,
                                 device=DEV)
    groups = bmod.share_groups(wl.block_tables, wl.context_lens, 3)
    members, tiles, start = bmod.group_tiles(wl.block_tables, wl.context_lens, groups,
                                             wl.block_size, 3)
    lens_d = torch.from_numpy(wl.context_lens).to(DEV)
    out = torch.empty_like(wl.q)

    def call(mem, til, sta, part_tiles=0, max_group_tiles=0):
        pk.paged_attention_decode_grouped(
            out, wl.q, wl.k_cache, wl.v_cache, lens_d, torch.from_numpy(mem).to(DEV),
            torch.from_numpy(til).to(DEV), torch.from_numpy(sta).to(DEV), wl.scale,
            int(wl.context_lens.max()), part_tiles=part_tiles, max_group_tiles=max_group_tiles)

    call(members, tiles, start)   # valid
    torch.cuda.synchronize()
    cases = []
    t = tiles.copy()
    t[1, 2] = 0                    # a tile with no member: member 0 loses tile 1
    cases.append((members, t, start, "has no entry"))
    t = tiles.copy()
    t[0, 0] = wl.num_blocks        # outside the pool
    cases.append((members, t, start, "outside the pool"))
    m = members.copy()
    m[1, 0] = m[0, 0]              # one sequence in two groups
    cases.append((m, tiles, start, "two groups"))
    for mem, til, sta, match in cases:
        with pytest.raises(pk.PagedKVError) as e:
            call(mem, til, sta)
        assert e.value.status == -1 and match in str(e.value), str(e.value)
    longest = int(np.diff(start).max())
    call(members, tiles, start, part_tiles=2, max_group_tiles=longest)   # valid
    torch.cuda.synchronize()
    with pytest.raises(pk.PagedKVError) as e:   # a bound below the longest group
        call(members, tiles, start, part_tiles=2, max_group_tiles=longest - 3)
    assert e.value.status == -1 and "max_group_tiles" in str(e.value), str(e.value)


@pytest.mark.parametrize("part_tiles", [0, 3])
@pytest.mark.parametrize("dtype,hq,hkv,hd,bs,width,build", [
    (torch.float16, 8, 8, 128, 16, 8, "sharing"),
    (torch.bfloat16, 16, 4, 128, 32, 4, "beam"),
    (torch.bfloat16, 6, 2, 64, 16, 5, "beam"),
])
def test_grouped_over_e4m3_codes(dtype, hq, hkv, hd, bs, width, build, part_tiles):
    """The 8-bit cache: random E4M3 codes in every owned slot, NaN codes in every
    slot no sequence owns, against the oracle's decode over dequantised codes."""
    import math
    from oracle import fp8
    say("grouped e4m3", dtype, hq, hkv, hd, bs, width, build, part_tiles)
    if build == "sharing":
        wl = workloads.build_sharing(num_prompts=4, fanout=width, prompt_len=60, max_gen=40,
                                     num_heads=hq, head_dim=hd, block_size=bs, num_blocks=512,
                                     seed=70 + hd, tensors=False)
    else:
        wl = workloads.build_beam_search(num_requests=4, beam_width=width, prompt_lens=(5, 90),
                                         steps=25, num_q_heads=hq, num_kv_heads=hkv, head_dim=hd,
                                         block_size=bs, num_blocks=512, seed=80 + hq,
                                         tensors=False)
    rng = np.random.default_rng(hq + hd + bs)
    nb, h = wl.num_blocks, wl.num_kv_heads
    kc = rng.integers(0, 256, (nb, h, bs, hd)).astype(np.uint8)
    vc = rng.integers(0, 256, (nb, h, bs, hd)).astype(np.uint8)
    for c in (kc, vc):
        c[(c & 0x7F) == 0x7F] = 0x00
    used = np.zeros((nb, bs), bool)
    for s in range(wl.num_seqs):
        for t in range(int(wl.context_lens[s])):
            used[wl.block_tables[s][t // bs], t % bs] = True
    kc[~used[:, None, :, None].repeat(h, 1).repeat(hd, 3)] = 0x7F
    vc[~used[:, None, :, None].repeat(h, 1).repeat(hd, 3)] = 0xFF
    q = torch.randn((wl.num_seqs, wl.num_q_heads, hd),
                    generator=torch.Generator().manual_seed(3)).to(dtype)
    k_scale, v_scale, scale = 1.0 / 96, 1.0 / 128, 1.0 / math.sqrt(hd)
    groups = bmod.share_groups(wl.block_tables, wl.context_lens, 16 // (wl.num_q_heads // h))
    members, tiles, start, longest = _lists(wl.block_tables, wl.context_lens, groups, bs,
                                            16 // (wl.num_q_heads // h))
    out = torch.full((wl.num_seqs, wl.num_q_heads, hd), float("nan"), dtype=dtype, device=DEV)
    pk.paged_attention_decode_grouped(out, q.to(DEV), torch.from_numpy(kc).to(DEV),
                                      torch.from_numpy(vc).to(DEV),
                                      torch.from_numpy(wl.context_lens).to(DEV), members, tiles,
                                      start, scale, int(wl.context_lens.max()),
                                      part_tiles=part_tiles, max_group_tiles=longest,
                                      k_scale=k_scale, v_scale=v_scale)
    torch.cuda.synchronize()
    want = fp8.decode_fp8(q, kc, vc, wl.block_tables, wl.context_lens, scale, k_scale, v_scale, h)
    got = out.cpu().double().numpy()
    assert np.isfinite(got).all()
    err = float(np.abs(got - want).max())
    assert err <= TOL[dtype], f"max abs err {err}"


@pytest.mark.parametrize("name", ["sharing_fp16", "beam_search_fp16"])
def test_full_size_grouped_over_e4m3(name):
    """The sharing and beam batches at full size with 8-bit pools (every slot
    quantised by the library's cache write), decoded by the grouped call;
    sampled sequences (the longest, the shortest, seeded others; all heads)
    against the oracle's decode over the same codes."""
    from oracle import fp8
    from gpu_helpers import compact_pool
    say("full-size grouped e4m3 build", name)
    wl = workloads.make(name, device=DEV)
    nb, hkv, bs, hd = wl.k_cache.shape
    k_scale = float(wl.k_cache.abs().amax().float()) / 448
    v_scale = float(wl.v_cache.abs().amax().float()) / 448
    kc = torch.empty((nb, hkv, bs, hd), dtype=torch.uint8, device=DEV)
    vc = torch.empty_like(kc)
    for b0 in range(0, nb, 1024):
        b1 = min(nb, b0 + 1024)
        rk = wl.k_cache[b0:b1].permute(0, 2, 1, 3).reshape(-1, hkv, hd).contiguous()
        rv = wl.v_cache[b0:b1].permute(0, 2, 1, 3).reshape(-1, hkv, hd).contiguous()
        pk.reshape_and_cache_fp8(rk, rv, kc, vc,
                                 torch.arange(b0 * bs, b1 * bs, dtype=torch.int64, device=DEV),
                                 k_scale, v_scale)
    torch.cuda.synchronize()
    L = wl.context_lens
    rng = np.random.default_rng(wl.seed)
    seqs = sorted({int(np.argmax(L)), int(np.argmin(L))} |
                  {int(s) for s in rng.choice(wl.num_seqs, 6, replace=False)})
    wl_codes = workloads.Workload(**{**wl.__dict__, "k_cache": kc, "v_cache": vc})
    kcs, vcs, tables = compact_pool(wl_codes, seqs)
    want = fp8.decode_fp8(wl.q.cpu(), kcs.numpy(), vcs.numpy(), tables, L, wl.scale, k_scale,
                          v_scale, wl.num_kv_heads, seqs=seqs)
    groups = bmod.share_groups(wl.block_tables, L, 16)
    members, tiles, start, longest = _lists(wl.block_tables, L, groups, bs, 16)
    for part_tiles in (0, 32):
        say("full-size grouped e4m3 decode", name, part_tiles)
        out = torch.empty_like(wl.q)
        pk.paged_attention_decode_grouped(out, wl.q, kc, vc, torch.from_numpy(L).to(DEV),
                                          members, tiles, start, wl.scale, wl.max_context_len,
                                          part_tiles=part_tiles, max_group_tiles=longest,
                                          k_scale=k_scale, v_scale=v_scale)
        torch.cuda.synchronize()
        got = out.cpu().double().numpy()[seqs]
        assert np.isfinite(got).all()
        err = float(np.abs(got - want[seqs]).max())
        assert err <= TOL[wl.dtype], f"{name} parts {part_tiles}: max abs err {err}"


# ------------------------------------------------ lists built on the device

def _device_lists(tables, lens, groups, bs, max_members, max_len, cap=None):
    members = np.full((len(groups), max_members), -1, np.int32)
    for j, g in enumerate(groups):
        members[j, :len(g)] = g
    t = torch.from_numpy(np.ascontiguousarray(tables, dtype=np.int32)).to(DEV)
    l = torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).to(DEV)
    m = torch.from_numpy(members).to(DEV)
    tiles = None if cap is None else torch.full((cap, 4), -7, dtype=torch.int32, device=DEV)
    tiles, start, end = pk.group_tiles(t, l, m, bs, max_len, tiles=tiles)
    torch.cuda.synchronize()
    return members, tiles.cpu().numpy(), start.cpu().numpy(), end.cpu().numpy()


def _same_as_host(tables, lens, groups, bs, max_members, max_len):
    hm, ht, hs = bmod.group_tiles(tables, lens, groups, bs, max_members)
    dm, dt, ds, de = _device_lists(tables, lens, groups, bs, max_members, max_len)
    assert np.array_equal(hm, dm)
    for j in range(len(groups)):
        assert np.array_equal(ht[hs[j]:hs[j + 1]], dt[ds[j]:de[j]]), j


@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("build", ["sharing", "beam", "unrelated"])
def test_device_lists_equal_host_lists(build, bs):
    say("device lists", build, bs)
    if build == "sharing":
        wl = workloads.build_sharing(num_prompts=7, fanout=6, prompt_len=90, max_gen=70,
                                     block_size=bs, num_blocks=1024, seed=bs, tensors=False)
    elif build == "beam":
        wl = workloads.build_beam_search(num_requests=6, beam_width=5, prompt_lens=(3, 120),
                                         steps=30, block_size=bs, num_blocks=1024, seed=bs + 1,
                                         tensors=False)
    else:
        rng = np.random.default_rng(bs)
        lens = np.r_[0, 1, 15, 16, 17, rng.integers(0, 400, 35)].astype(np.int32)
        width = -(-400 // bs) + 1
        tables = rng.integers(-3, 5000, (len(lens), width)).astype(np.int32)  # any entries
        order = rng.permutation(len(lens))
        groups = [list(map(int, order[i:i + 3])) for i in range(0, len(order), 3)]
        _same_as_host(tables, lens, groups, bs, 3, 400)
        return
    for mm in (16, 4):
        groups = bmod.share_groups(wl.block_tables, wl.context_lens, mm)
        _same_as_host(wl.block_tables, wl.context_lens, groups, bs, mm,
                      int(wl.context_lens.max()))


def test_device_lists_many_groups_empty_groups_and_capacity():
    say("device lists: many groups")
    rng = np.random.default_rng(9)
    n = 4096
    lens = rng.integers(0, 70, n).astype(np.int32)
    lens[::7] = 0                                   # empty groups, some at the ends
    lens[-1] = 0
    tables = rng.integers(0, 100000, (n, 5)).astype(np.int32)
    groups = [[s] for s in range(n)]
    _same_as_host(tables, lens, groups, 16, 1, 80)
    pairs = [[s, s + 1] for s in range(0, 600, 2)]          # 2 members in 16 places
    _same_as_host(tables, lens, pairs, 16, 16, 80)
    with pytest.raises(pk.PagedKVError) as e:               # a short list buffer
        _device_lists(tables, lens, groups, 16, 1, 80, cap=n * 5 - 1)
    assert e.value.status == -3


def test_grouped_decode_from_device_lists():
    say("grouped decode from device lists")
    wl = workloads.make("sharing_fp16", device=DEV)
    groups = bmod.share_groups(wl.block_tables, wl.context_lens, 16)
    host = _lists(wl.block_tables, wl.context_lens, groups, wl.block_size, 16)
    tiles_d, start_d, end_d = pk.group_tiles(
        torch.from_numpy(wl.block_tables).to(DEV), torch.from_numpy(wl.context_lens).to(DEV),
        host[0], wl.block_size, wl.max_context_len)
    lens_d = torch.from_numpy(wl.context_lens).to(DEV)
    a = _grouped(wl.q, wl.k_cache, wl.v_cache, lens_d, host, wl.scale, wl.max_context_len)
    for part_tiles in (0, 32):
        b = torch.full_like(wl.q, float("nan"))
        pk.paged_attention_decode_grouped(b, wl.q, wl.k_cache, wl.v_cache, lens_d, host[0],
                                          tiles_d, start_d, wl.scale, wl.max_context_len,
                                          part_tiles=part_tiles, max_group_tiles=host[3],
                                          group_tile_end=end_d)
        torch.cuda.synchronize()
        if part_tiles == 0:
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        else:
            assert float((a.float() - b.float()).abs().max()) <= TOL[wl.dtype]


def test_debug_checks_device_built_lists(monkeypatch):
    """PKV_DEBUG=1 with per-group start/end offsets (the device builder's form):
    valid lists pass, an end before its start or a tile missing from a group
    is rejected before anything runs."""
    say("grouped debug checks, start/end form")
    monkeypatch.setenv("PKV_DEBUG", "1")
    wl = workloads.build_sharing(dtype=torch.float16, num_prompts=3, fanout=4, prompt_len=50,
                                 max_gen=20, num_heads=2, head_dim=64, num_blocks=128, seed=4,
                                 device=DEV)
    groups = bmod.share_groups(wl.block_tables, wl.context_lens, 4)
    members = np.full((len(groups), 4), -1, np.int32)
    for j, g in enumerate(groups):
        members[j, :len(g)] = g
    m = torch.from_numpy(members).to(DEV)
    lens = torch.from_numpy(wl.context_lens).to(DEV)
    tiles, start, end = pk.group_tiles(torch.from_numpy(wl.block_tables).to(DEV), lens, m,
                                       wl.block_size, wl.max_context_len)
    out = torch.empty_like(wl.q)

    def call(end_arr):
        pk.paged_attention_decode_grouped(out, wl.q, wl.k_cache, wl.v_cache, lens, m, tiles,
                                          start, wl.scale, wl.max_context_len,
                                          group_tile_end=end_arr)

    call(end)
    torch.cuda.synchronize()
    want = oracle.decode(wl.q.cpu(), wl.k_cache.cpu(), wl.v_cache.cpu(), wl.block_tables,
                         wl.context_lens, wl.scale, wl.num_kv_heads)
    assert max_err(out, want) <= TOL[torch.float16]
    bad = end.clone()
    bad[1] = start[1] - 1                       # end before start
    with pytest.raises(pk.PagedKVError) as e:
        call(bad)
    assert e.value.status == -1 and "outside" in str(e.value), str(e.value)
    short = end.clone()
    short[0] -= 1                               # group 0 loses its last row
    with pytest.raises(pk.PagedKVError) as e:
        call(short)
    assert e.value.status == -1 and "no entry" in str(e.value), str(e.value)
