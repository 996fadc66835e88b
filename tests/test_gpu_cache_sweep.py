"""Seeded random cache writes and block copies against the oracle, bit for
bit over the whole cache: dtype (and the quantising E4M3 write), head dim,
block size, KV heads, pool size, a random distinct set of slots with some
skipped (negative) entries, and copy pairs with distinct destinations that
are never sources; the caches start from random bit patterns, so slots the
calls must not touch are checked too."""

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, say
from oracle import cache_ops
from oracle import fp8 as ofp8
from paged_kv_cache_389_amd import _native as pk

pytestmark = pytest.mark.gpu

DTYPES = (torch.float32, torch.float16, torch.bfloat16)
BITS = {torch.float32: torch.int32, torch.float16: torch.int16, torch.bfloat16: torch.int16}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")


def cache_case(i):
    rng = np.random.default_rng(13000 + i)
    dtype = DTYPES[i % 3]
    fp8 = i % 4 == 3
    hd = (64, 128, 256)[int(rng.integers(0, 3))]
    bs = (8, 16, 32)[int(rng.integers(0, 3))]
    hkv = int(rng.integers(1, 9))
    nb = int(rng.integers(4, 200))
    n_tok = int(rng.integers(0, min(nb * bs, 600) + 1))
    slots = rng.choice(nb * bs, n_tok, replace=False).astype(np.int64)
    slots[rng.random(n_tok) < 0.1] = -1   # skipped
    n_pairs = int(rng.integers(0, nb // 2 + 1))
    perm = rng.permutation(nb)
    pairs = np.stack([perm[:n_pairs], perm[n_pairs:2 * n_pairs]], axis=1).astype(np.int64)
    return rng, dtype, fp8, hd, bs, hkv, nb, slots, pairs


def _random_cache(rng, shape, dtype, fp8):
    if fp8:
        return torch.from_numpy(rng.integers(0, 256, shape).astype(np.uint8))
    if dtype == torch.float32:   # finite random values: bit compare is exact either way
        return torch.from_numpy(rng.standard_normal(shape).astype(np.float32))
    bits = rng.integers(-(1 << 15), 1 << 15, shape).astype(np.int16)
    return torch.from_numpy(bits).view(dtype)


@pytest.mark.parametrize("i", range(16))
def test_cache_ops_random_sweep(i):
    rng, dtype, fp8, hd, bs, hkv, nb, slots, pairs = cache_case(i)
    say("cache sweep", i, dtype, "fp8" if fp8 else "plain", hd, bs, hkv, nb, len(slots), len(pairs))
    shape = (nb, hkv, bs, hd)
    kc = _random_cache(rng, shape, dtype, fp8)
    vc = _random_cache(rng, shape, dtype, fp8)
    k = torch.from_numpy(rng.standard_normal((len(slots), hkv, hd)) * 4).to(dtype)
    v = torch.from_numpy(rng.standard_normal((len(slots), hkv, hd)) * 4).to(dtype)
    kd, vd = kc.clone().to(DEV), vc.clone().to(DEV)
    slots_d = torch.from_numpy(slots).to(DEV)
    if fp8:
        k_scale, v_scale = float(k.abs().max()) / 448 + 1e-3, float(v.abs().max()) / 448 + 1e-3
        pk.reshape_and_cache_fp8(k.to(DEV), v.to(DEV), kd, vd, slots_d, k_scale, v_scale)
        want_k, want_v = kc.numpy().copy(), vc.numpy().copy()
        ofp8.reshape_and_cache_fp8(k, v, want_k, want_v, slots, k_scale, v_scale)
    else:
        pk.reshape_and_cache(k.to(DEV), v.to(DEV), kd, vd, slots_d)
        want_k, want_v = kc.clone(), vc.clone()
        cache_ops.reshape_and_cache(k, v, want_k, want_v, slots)
        want_k, want_v = want_k.view(BITS[dtype]).numpy(), want_v.view(BITS[dtype]).numpy()
    torch.cuda.synchronize()
    view = (lambda t: t.cpu().numpy()) if fp8 else (lambda t: t.cpu().view(BITS[dtype]).numpy())
    assert np.array_equal(view(kd), want_k)
    assert np.array_equal(view(vd), want_v)
    # then the copy-on-write copies of whole blocks
    if len(pairs):
        pk.copy_blocks(kd, vd, torch.from_numpy(pairs).to(DEV))
        cache_ops.copy_blocks(want_k, want_v, pairs)
        torch.cuda.synchronize()
        assert np.array_equal(view(kd), want_k)
        assert np.array_equal(view(vd), want_v)
