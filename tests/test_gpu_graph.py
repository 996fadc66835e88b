"""The decode step captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: copy_blocks -> reshape_and_cache -> paged_attention_decode on the
planned grid with a split (planning kernel, partition merge) and on the
direct grid.  Every replay, with eager work and synchronisations between
replays, gives bit-identical results to the eager calls; the library enqueues
no memset and allocates nothing, so the calls are capturable as they are."""

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, INT_VIEW, say
from paged_kv_cache_389_amd import _native as pk
from paged_kv_cache_389_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")


@pytest.mark.parametrize("grid,partition", [(pk.GRID_PLANNED, 512), (pk.GRID_DIRECT, 0)])
def test_captured_step_replays_match_eager(grid, partition):
    say("graph replay", grid, partition)
    wl = workloads.make("llama3_8b_gqa_bf16", device=DEV, num_seqs=48, num_blocks=16384)
    tables = torch.from_numpy(wl.block_tables).to(DEV)
    lens = torch.from_numpy(wl.context_lens).to(DEV)
    st = wl.step
    slots = torch.from_numpy(st.slot_mapping).to(DEV)
    pairs = torch.tensor([[5, 6], [7, 8]], dtype=torch.int64, device=DEV)
    k0, v0 = wl.k_cache.clone(), wl.v_cache.clone()
    ws = torch.empty(max(1, pk.workspace_bytes(
        wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size,
        tables.shape[1], wl.max_context_len, wl.dtype, partition, 0, grid)),
        dtype=torch.uint8, device=DEV)
    out = torch.empty_like(wl.q)

    def step():
        pk.copy_blocks(wl.k_cache, wl.v_cache, pairs)
        pk.reshape_and_cache(st.new_k, st.new_v, wl.k_cache, wl.v_cache, slots)
        pk.paged_attention_decode(out, wl.q, wl.k_cache, wl.v_cache, tables, lens, wl.scale,
                                  wl.max_context_len, workspace=ws, partition_tokens=partition,
                                  grid=grid)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    k_eager = wl.k_cache.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        wl.k_cache.copy_(k0)
        wl.v_cache.copy_(v0)
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.synchronize()
    iv = INT_VIEW[wl.dtype]
    for r in range(4):
        out.fill_(float("nan"))            # eager work between replays
        wl.k_cache.copy_(k0)
        wl.v_cache.copy_(v0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(iv), eager.view(iv)), f"replay {r} differs"
        assert torch.equal(wl.k_cache.view(iv), k_eager.view(iv)), f"replay {r}: K cache differs"


@pytest.mark.parametrize("part_tiles", [0, 24])
def test_captured_grouped_decode_replays_match_eager(part_tiles):
    """The grouped decode (and, with parts, its merge kernel) captured and
    replayed: every replay bit-identical to the eager call."""
    from paged_kv_cache_389_amd import block_manager as bmod
    say("graph replay grouped", part_tiles)
    wl = workloads.build_sharing(dtype=torch.float16, num_prompts=6, fanout=8, prompt_len=300,
                                 max_gen=60, num_heads=8, head_dim=128, num_blocks=2048, seed=21,
                                 device=DEV)
    groups = bmod.share_groups(wl.block_tables, wl.context_lens, 16)
    members, tiles, start = bmod.group_tiles(wl.block_tables, wl.context_lens, groups,
                                             wl.block_size, 16)
    longest = int(np.diff(start).max())
    lists = [torch.from_numpy(x).to(DEV) for x in (members, tiles, start)]
    lens = torch.from_numpy(wl.context_lens).to(DEV)
    ws = torch.empty(max(1, pk.grouped_workspace_bytes(len(groups), wl.num_kv_heads, wl.head_dim,
                                                       part_tiles, longest)),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty_like(wl.q)

    def call():
        pk.paged_attention_decode_grouped(out, wl.q, wl.k_cache, wl.v_cache, lens, *lists,
                                          wl.scale, wl.max_context_len, part_tiles=part_tiles,
                                          max_group_tiles=longest, workspace=ws)

    call()
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            call()
    torch.cuda.synchronize()
    iv = INT_VIEW[wl.dtype]
    for r in range(4):
        out.fill_(float("nan"))
        ws.fill_(255)                      # the part states need no initialisation
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(iv), eager.view(iv)), f"replay {r} differs"
