"""A KV pool larger than 4 GiB per cache, with every block the sequences use
near its top, so that every kernel's block offsets pass 32 bits: decode
(both kernels), the cache write, copy_blocks and prefill, against the oracle
on the blocks involved (copied out and renumbered)."""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, TOL, decode_gpu, say
from paged_kv_cache_389_amd import _native as pk

pytestmark = pytest.mark.gpu

NB, HKV, BS, HD = 150_000, 8, 16, 128        # 32 KiB per block and cache: 4.6 GiB per pool


@pytest.fixture(scope="module")
def pools():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    say("large pool alloc", NB)
    k = torch.empty((NB, HKV, BS, HD), dtype=torch.bfloat16, device=DEV)
    v = torch.empty_like(k)
    assert k.numel() * k.element_size() > 4 << 30
    yield k, v
    del k, v
    torch.cuda.empty_cache()


def test_top_of_a_large_pool(pools):
    k, v = pools
    rng = np.random.default_rng(77)
    g = torch.Generator(device=DEV).manual_seed(77)
    lens = np.array([300, 33, 1, 129], np.int32)
    nblk = -(-lens // BS)
    used = NB - 1 - rng.permutation(200)[:int(nblk.sum()) + 2]   # blocks in the top 200
    tables = np.zeros((4, int(nblk.max())), np.int32)
    at = 0
    for s, n in enumerate(nblk):
        tables[s, :n] = used[at:at + n]
        at += n
    spare_src, spare_dst = int(used[at]), int(used[at + 1])
    idx = torch.from_numpy(used.astype(np.int64)).to(DEV)
    k[idx] = torch.randn((len(used), HKV, BS, HD), generator=g, device=DEV).to(torch.bfloat16)
    v[idx] = torch.randn((len(used), HKV, BS, HD), generator=g, device=DEV).to(torch.bfloat16)

    # cache write into the last slot of sequence 0 and a copy between top blocks
    say("large pool writes")
    new = torch.randn((1, HKV, HD), generator=g, device=DEV).to(torch.bfloat16)
    slot = torch.tensor([int(tables[0, (lens[0] - 1) // BS]) * BS + (lens[0] - 1) % BS],
                        dtype=torch.int64, device=DEV)
    pk.reshape_and_cache(new, new, k, v, slot)
    pk.copy_blocks(k, v, torch.tensor([[spare_src, spare_dst]], dtype=torch.int64, device=DEV))
    torch.cuda.synchronize()
    s_blk, s_off = divmod(int(slot), BS)
    assert torch.equal(k[s_blk, :, s_off].view(torch.int16), new[0].view(torch.int16))
    assert torch.equal(k[spare_dst].view(torch.int16), k[spare_src].view(torch.int16))

    # the oracle reads the used blocks only, renumbered 0..n-1
    remap = {int(b): i for i, b in enumerate(used)}
    kc = k[idx].cpu()
    vc = v[idx].cpu()
    tab_small = np.vectorize(lambda b: remap.get(int(b), 0))(tables)
    tab = torch.from_numpy(tables).to(DEV)
    L = torch.from_numpy(lens).to(DEV)
    for hq, path in ((32, pk.PATH_MFMA), (8, pk.PATH_VALU)):
        say("large pool decode", hq, path)
        q = torch.randn((4, hq, HD), generator=g, device=DEV).to(torch.bfloat16)
        got = decode_gpu(q, k, v, tab, L, 1 / math.sqrt(HD), path=path)
        want = oracle.decode(q.cpu(), kc, vc, tab_small, lens, 1 / math.sqrt(HD), HKV)
        assert float(np.abs(got.cpu().double().numpy() - want).max()) <= TOL[torch.bfloat16]

    say("large pool prefill")
    qs = np.array([0, 40, 73, 74, 203], np.int32)        # chunks of 40, 33 (all), 1, 129 (all)
    qp = torch.randn((203, 32, HD), generator=g, device=DEV).to(torch.bfloat16)
    out = torch.empty_like(qp)
    pk.paged_attention_prefill(out, qp, k, v, tab, L, torch.from_numpy(qs).to(DEV),
                               1 / math.sqrt(HD), 129, int(lens.max()))
    torch.cuda.synchronize()
    rows = [0, 39, 40, 72, 73, 74, 150, 202]
    want = oracle.prefill(qp.cpu(), kc, vc, tab_small, lens, qs, 1 / math.sqrt(HD), HKV, rows=rows)
    got = out.cpu().double().numpy()[rows]
    assert float(np.abs(got - want[rows]).max()) <= TOL[torch.bfloat16]
