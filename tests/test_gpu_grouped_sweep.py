"""Seeded random batches through the grouped decode against the float64
oracle: the workload kind (forked prompts, beam search, requests sharing a
system prompt), query type, head layout, head dim, block size, members per
group, parts and 16-bit or E4M3 cache are drawn per case; every slot no
sequence owns holds NaN (or a NaN code).  Bar: max-abs 2e-2."""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, TOL, max_err, say
from oracle import fp8 as ofp8
from paged_kv_cache_389_amd import _native as pk
from paged_kv_cache_389_amd import block_manager as bmod
from paged_kv_cache_389_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")


def grouped_case(i):
    """Case i's workload (host tensors only) and call parameters."""
    rng = np.random.default_rng(11000 + i)
    kind = ("sharing", "beam", "system")[i % 3]
    dtype = (torch.float16, torch.bfloat16)[(i // 3) % 2]
    fp8 = i % 4 == 1
    hd = (64, 128)[int(rng.integers(0, 2))]
    bs = (16, 32)[int(rng.integers(0, 2))]
    seed = int(rng.integers(0, 1 << 20))
    if kind == "sharing":   # multi-head: up to 16 forks per group
        heads = int(rng.integers(1, 9))
        fanout = int(rng.integers(2, 17))
        wl = workloads.build_sharing(num_prompts=int(rng.integers(1, 6)), fanout=fanout,
                                     prompt_len=int(rng.integers(1, 150)), max_gen=int(rng.integers(0, 60)),
                                     num_heads=heads, head_dim=hd, block_size=bs, num_blocks=1024,
                                     seed=seed, tensors=False)
        g = 1
    else:
        hkv = int(rng.integers(1, 5))
        g = (1, 2, 3, 4, 8)[int(rng.integers(0, 5))]
        if kind == "beam":
            wl = workloads.build_beam_search(num_requests=int(rng.integers(1, 6)),
                                             beam_width=int(rng.integers(2, 16 // g + 1)),
                                             prompt_lens=(1, 120), steps=int(rng.integers(1, 40)),
                                             num_q_heads=hkv * g, num_kv_heads=hkv, head_dim=hd,
                                             block_size=bs, num_blocks=1024, seed=seed,
                                             tensors=False)
        else:
            wl = workloads.build_system_prompt(num_prefixes=int(rng.integers(1, 4)),
                                               requests_per_prefix=int(rng.integers(2, 10)),
                                               prefix_blocks=(1, 6), own_prompt=(1, 80),
                                               max_gen=int(rng.integers(0, 30)), num_q_heads=hkv * g,
                                               num_kv_heads=hkv, head_dim=hd, block_size=bs,
                                               num_blocks=1024, seed=seed, tensors=False)
    max_members = 16 // g if rng.random() < 0.7 else int(rng.integers(1, 16 // g + 1))
    part_tiles = (0, 0, 2, 5, 16)[int(rng.integers(0, 5))]
    return rng, kind, dtype, fp8, wl, max_members, part_tiles


@pytest.mark.parametrize("i", range(18))
def test_grouped_random_sweep(i):
    rng, kind, dtype, fp8, wl, max_members, part_tiles = grouped_case(i)
    bs, hd, h = wl.block_size, wl.head_dim, wl.num_kv_heads
    say("grouped sweep", i, kind, dtype, "fp8" if fp8 else "plain", wl.num_q_heads, h, hd, bs,
        "seqs", wl.num_seqs, "members", max_members, "parts", part_tiles)
    nb = wl.num_blocks
    used = np.zeros((nb, bs), bool)
    for s in range(wl.num_seqs):
        for t in range(int(wl.context_lens[s])):
            used[wl.block_tables[s][t // bs], t % bs] = True
    unowned = ~used[:, None, :, None].repeat(h, 1).repeat(hd, 3)
    if fp8:
        kc = rng.integers(0, 256, (nb, h, bs, hd)).astype(np.uint8)
        vc = rng.integers(0, 256, (nb, h, bs, hd)).astype(np.uint8)
        for c in (kc, vc):
            c[(c & 0x7F) == 0x7F] = 0x00
        kc[unowned] = 0x7F
        vc[unowned] = 0xFF
        kt, vt = torch.from_numpy(kc), torch.from_numpy(vc)
    else:
        kp = rng.standard_normal((nb, h, bs, hd))
        vp = rng.standard_normal((nb, h, bs, hd))
        kp[unowned] = np.nan
        vp[unowned] = np.nan
        kt, vt = torch.from_numpy(kp).to(dtype), torch.from_numpy(vp).to(dtype)
    q = torch.from_numpy(rng.standard_normal((wl.num_seqs, wl.num_q_heads, hd))).to(dtype)
    scale = float(rng.uniform(0.5, 1.5)) / math.sqrt(hd)
    k_scale, v_scale = 1.0 / 96, 1.0 / 128
    groups = bmod.share_groups(wl.block_tables, wl.context_lens, max_members)
    members, tiles, start = bmod.group_tiles(wl.block_tables, wl.context_lens, groups, bs,
                                             max_members)
    if tiles.shape[0] == 0:
        tiles = np.zeros((1, 4), np.int32)
    longest = int(np.diff(start).max(initial=0))
    out = torch.full((wl.num_seqs, wl.num_q_heads, hd), float("nan"), dtype=dtype, device=DEV)
    extra = dict(k_scale=k_scale, v_scale=v_scale) if fp8 else {}
    pk.paged_attention_decode_grouped(out, q.to(DEV), kt.to(DEV), vt.to(DEV),
                                      torch.from_numpy(wl.context_lens).to(DEV),
                                      torch.from_numpy(members).to(DEV),
                                      torch.from_numpy(tiles).to(DEV),
                                      torch.from_numpy(start).to(DEV), scale,
                                      int(wl.context_lens.max()), part_tiles=part_tiles,
                                      max_group_tiles=longest, **extra)
    torch.cuda.synchronize()
    if fp8:
        want = ofp8.decode_fp8(q, kc, vc, wl.block_tables, wl.context_lens, scale, k_scale, v_scale, h)
    else:
        want = oracle.decode(q, kt, vt, wl.block_tables, wl.context_lens, scale, h)
    got = out.cpu().double().numpy()
    assert np.isfinite(got).all()
    err = max_err(out, want)
    assert err <= TOL[dtype], f"max abs err {err}"
