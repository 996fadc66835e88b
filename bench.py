"""Benchmark of the paged decode hot path on one MI355X.

One step = the whole path over one batch: copy_blocks (the step's
copy-on-write pairs, if any) -> reshape_and_cache (the step's new tokens, if
any) -> paged_attention_decode over every sequence.  Inputs are synthetic,
seeded, and resident in HBM before the timed region.

Prints ONE JSON line.  ``value`` is whole-step throughput in algorithmic
bytes per second (GB/s): the K/V bytes the attention must read plus q, out,
tables, lengths and the cache writes.  ``roofline`` reports the attention
kernel's own achieved HBM bandwidth (the decode call's algorithmic bytes
over the kernel's average duration, timed with HIP events that the library
records around that launch on its stream) against the MI355X HBM3E peak of
8 TB/s, with the HBM bytes per launch that rocprofv3 counters measured
(``traffic``, from profiles/decode_traffic.json while the kernel sources
are unchanged, else null).  ``decode_ms`` times the whole decode call
(planning kernel and partition merge included) in a second pass of as many
steps after the timed one, so that its event markers stay out of the timed
steps.  ``cpu_baseline`` times the
float64 CPU oracle on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--sweep]
"""

import argparse
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
HOST_LINK_GBS = 64.0   # PCIe 5.0 x16, one direction
PREFILL_WORKLOADS = ("llama3_8b_prefill_bf16",)
GROUPABLE = ("sharing_fp16", "beam_search_fp16", "system_prompt_bf16")
DEFAULT_WORKLOAD = "opt13b_fp16"
DTYPE_NAME = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}
WORKLOAD_DESC = {
    "tiny_fp32": dict(num_seqs=4, heads="4/4", head_dim=64, block_size=16,
                      context_lens="U[1,64]", pool_blocks=32),
    "opt13b_fp16": dict(num_seqs=64, heads="40/40", head_dim=128, block_size=16,
                        context_lens="U[128,2048]", pool_blocks=8192),
    "llama3_8b_gqa_bf16": dict(num_seqs=256, heads="32/8", head_dim=128, block_size=16,
                               context_lens="logU[16,4096]", pool_blocks=32768,
                               new_token_per_seq=True),
    "long_context_gqa_bf16": dict(num_seqs=8, heads="64/8", head_dim=128, block_size=32,
                                  context_lens="U[16384,32768]", pool_blocks=12288,
                                  key_outliers="1% x8"),
    "sharing_fp16": dict(num_seqs=256, prompts=32, fanout=8, heads="32/32", head_dim=128,
                         block_size=16, context_lens="1024+U[1,15]+U[0,256]",
                         pool_blocks=8192),
    "system_prompt_bf16": dict(num_seqs=128, system_prompts=4, requests_per_prompt=32,
                               heads="32/8", head_dim=128, block_size=16,
                               context_lens="prompt 16*U[32,127]+U[1,15] (cached, shared) + "
                                            "own U[16,512] + generated U[0,64]",
                               pool_blocks=8192),
    "beam_search_fp16": dict(num_seqs=128, requests=16, beam_width=8, heads="32/32",
                             head_dim=128, block_size=16,
                             context_lens="prompt U[256,1024] + 64 beam steps",
                             pool_blocks=8192, timed_step="step 64 (its copy-on-write pairs, "
                                                          "128 new tokens, decode)"),
}


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD,
                   choices=sorted(WORKLOAD_DESC) + sorted(PREFILL_WORKLOADS))
    p.add_argument("--sweep", action="store_true", help="one line per workload")
    p.add_argument("--partition", type=int, default=0, help="tokens per partition (0 = auto)")
    p.add_argument("--path", type=int, default=0, help="0 auto, 1 VALU, 2 MFMA, 3 contiguous")
    p.add_argument("--grid", type=int, default=0, help="0 auto, 1 direct, 2 planned")
    p.add_argument("--kv-cache", default="auto", choices=["auto", "e4m3"],
                   help="e4m3: quantise the pools to 8-bit codes and time the 8-bit path")
    p.add_argument("--placement", default="random", choices=["random", "sequential"])
    p.add_argument("--grouped", action="store_true",
                   help="decode with the grouped call: sequences sharing their first block "
                        "(forks of one prompt) read each shared tile once")
    p.add_argument("--group-part", type=int, default=-1, metavar="TILES",
                   help="with --grouped: tiles per part (0 = whole groups, -1 = auto)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-budget-s", type=float, default=20.0)
    p.add_argument("--cpu-pool", type=int, default=min(16, len(os.sched_getaffinity(0))),
                   help="worker processes of the pooled oracle baseline (<= 1: none)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (counter calibration)")
    p.add_argument("--counters", metavar="OUT_JSON",
                   help="no run: turn rocprofv3 --pmc databases of FETCH_SIZE and WRITE_SIZE "
                        "(this workload, then the copy calibration) into HBM bytes per launch, "
                        "merged into OUT_JSON")
    p.add_argument("--fetch-db")
    p.add_argument("--write-db")
    p.add_argument("--cal-fetch-db")
    p.add_argument("--cal-write-db")
    p.add_argument("--cal-mib", type=int, default=1024)
    p.add_argument("--swap", type=int, default=0, metavar="BLOCKS",
                   help="measure swap_blocks of this many K+V block pairs each way instead")
    p.add_argument("--ceiling", action="store_true",
                   help="only the reference reads (stream and block gather): the practical "
                        "bandwidth ceiling")
    p.add_argument("--quick", action="store_true",
                   help="the headline line alone (no per-config, paging-control or ceiling "
                        "objects)")
    return p.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")


def kernel_sources_digest():
    """sha256 over the HIP sources of the library's path kernels (names and
    bytes; the reference reads of ceiling.hip are left out): counter figures
    are only used while the kernels they were taken on are built."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "paged_kv_cache_389_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h")) and f != "ceiling.hip":
            h.update(f.encode())
            with open(os.path.join(d, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(name):
    """HBM bytes per launch of the attention kernel from the committed
    counter summary, or None if there is none for this workload or the
    kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != kernel_sources_digest():
        return None
    w = rec.get("workloads", {}).get(name)
    return None if w is None else w.get("hbm_bytes_per_launch")


def _counter_means(db):
    """{(kernel name, counter): mean per dispatch} from a rocprofv3 database."""
    import glob
    import sqlite3
    files = [db] if db.endswith(".db") else glob.glob(os.path.join(db, "**", "*.db"),
                                                       recursive=True)
    acc = {}
    for f in files:
        con = sqlite3.connect(f)
        cols = [c[1] for c in con.execute("pragma table_info(counters_collection)")]
        ki, ci, vi = cols.index("kernel_name"), cols.index("counter_name"), cols.index("value")
        for r in con.execute("select * from counters_collection"):
            acc.setdefault((r[ki], r[ci]), []).append(float(r[vi]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def counters_to_traffic(args):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the attention kernel,
    each divided by what the same counter reads per byte of a plain copy of
    known size, give its HBM bytes per launch."""
    def pick(means, counter, want):
        rows = [(v, k) for (k, c), v in means.items() if c == counter and want(k)]
        if not rows:
            raise SystemExit(f"no {counter} rows")
        return max(rows)
    is_decode = lambda k: any(n in k for n in ("decode_mfma_kernel", "decode_valu_kernel",
                                               "prefill_mfma_kernel", "decode_grouped_kernel"))
    is_other = lambda k: "pkv::" not in k
    cal_bytes = args.cal_mib << 20
    f_fetch = pick(_counter_means(args.cal_fetch_db), "FETCH_SIZE", is_other)[0] * 1024 / cal_bytes
    f_write = pick(_counter_means(args.cal_write_db), "WRITE_SIZE", is_other)[0] * 1024 / cal_bytes
    # the attention kernel of the run: the one with the most fetched bytes;
    # its own WRITE_SIZE (another kernel of the run may write more)
    fetch, kname = pick(_counter_means(args.fetch_db), "FETCH_SIZE", is_decode)
    write, _ = pick(_counter_means(args.write_db), "WRITE_SIZE", lambda k: k == kname)
    from paged_kv_cache_389_amd import workloads
    kw = {"tensors": False} if args.workload in GROUPABLE else {}
    wl = workloads.make(args.workload, device="cpu", **kw)
    key = args.workload
    fp8 = args.kv_cache == "e4m3"
    logical = None
    if args.workload in PREFILL_WORKLOADS:
        alg = wl.min_bytes()
        if fp8:   # one byte per K/V element
            kv = (int(wl.context_lens.astype(np.int64).sum()) * 2 * wl.num_kv_heads *
                  wl.head_dim * wl.esize)
            alg -= kv - kv // wl.esize
    else:
        # the bytes the bench line's roofline is taken on (each shared slot once)
        alg, _ = roofline_bytes(wl, fp8, grouped_lists(wl, None) if args.grouped else None)
        logical = wl.decode_bytes() - ((wl.kv_bytes() - wl.kv_bytes() // wl.esize) if fp8 else 0)
    if fp8:
        key += "_kv_e4m3"
    if args.grouped:
        key += "_grouped"
    try:
        with open(args.counters) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        rec = {}
    if rec.get("sources_sha256") != kernel_sources_digest():
        rec = {"sources_sha256": kernel_sources_digest(), "workloads": {}}
    rec["calibration"] = {"copy_mib": args.cal_mib, "fetch_counter_per_byte": round(f_fetch, 4),
                          "write_counter_per_byte": round(f_write, 4)}
    rec["workloads"][key] = {
        "kernel": re.sub(r"\([^()]*\)$", "", kname), "fetch_kib_per_launch": round(fetch, 1),
        "write_kib_per_launch": round(write, 1),
        "hbm_bytes_per_launch": int(fetch * 1024 / f_fetch + write * 1024 / f_write),
        "alg_bytes_per_launch": alg}
    if logical is not None and logical != alg:
        rec["workloads"][key]["logical_bytes_per_launch"] = logical
    with open(args.counters, "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)
    print(json.dumps(rec["workloads"][key]))


def copy_calibration(mib, reps=5):
    """A plain device-to-device copy of a known size, run under rocprofv3
    --pmc to learn how FETCH_SIZE / WRITE_SIZE count bytes on this part."""
    n = mib << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "reps": reps}),
          flush=True)


def build_inputs(name, placement):
    from paged_kv_cache_389_amd import workloads
    kw = {"device": "cuda"}
    if placement != "random":
        kw["placement"] = placement
    wl = workloads.make(name, **kw)
    dev = dict(q=wl.q, k=wl.k_cache, v=wl.v_cache,
               tables=torch.from_numpy(wl.block_tables).cuda(),
               lens=torch.from_numpy(wl.context_lens).cuda(),
               out=torch.empty_like(wl.q))
    step = wl.step
    pairs = wl.meta.get("first_step_pairs") if wl.history else None
    if pairs is None and step is not None:
        pairs = step.copy_pairs
    dev["pairs"] = torch.from_numpy(np.ascontiguousarray(pairs)).cuda() \
        if pairs is not None and len(pairs) else None
    if step is not None and len(step.slot_mapping):
        dev["slots"] = torch.from_numpy(step.slot_mapping).cuda()
        dev["new_k"], dev["new_v"] = step.new_k, step.new_v
    else:
        dev["slots"] = None
    return wl, dev


def step_bytes(wl, dev):
    """Algorithmic bytes of the step: (decode, cache writes + copies).  With
    an 8-bit cache the K/V rows cost one byte per element (q and out keep
    the workload type) and the quantising write reads source rows and
    writes code rows."""
    row_src = wl.num_kv_heads * wl.head_dim * wl.esize
    row = wl.num_kv_heads * wl.head_dim * (1 if dev.get("kv_fp8") else wl.esize)
    n_tok = 0 if dev["slots"] is None else int(dev["slots"].numel())
    n_pair = 0 if dev["pairs"] is None else int(dev["pairs"].shape[0])
    writes = 2 * (n_tok * row_src + n_tok * row) + 8 * n_tok
    copies = 2 * (2 * n_pair * row * wl.block_size) + 16 * n_pair
    decode = wl.decode_bytes()
    if dev.get("kv_fp8"):
        decode -= wl.kv_bytes() - wl.kv_bytes() // wl.esize
    return decode, writes + copies


def quantise_pools(wl, dev):
    """Replace the workload's K/V pools by E4M3 code pools (one scale per
    cache: its largest magnitude over 448), written by the library's
    quantising cache write over every slot; set-up, not timed."""
    from paged_kv_cache_389_amd import _native as pk
    nb, hkv, bs, hd = dev["k"].shape
    k_scale = float(dev["k"].abs().amax().float()) / 448.0
    v_scale = float(dev["v"].abs().amax().float()) / 448.0
    kc = torch.empty((nb, hkv, bs, hd), dtype=torch.uint8, device="cuda")
    vc = torch.empty_like(kc)
    chunk = max(1, (1 << 27) // (hkv * hd * wl.esize) // bs)   # blocks per chunk (~128 MiB)
    for b0 in range(0, nb, chunk):
        b1 = min(nb, b0 + chunk)
        rows_k = dev["k"][b0:b1].permute(0, 2, 1, 3).reshape(-1, hkv, hd).contiguous()
        rows_v = dev["v"][b0:b1].permute(0, 2, 1, 3).reshape(-1, hkv, hd).contiguous()
        slots = torch.arange(b0 * bs, b1 * bs, dtype=torch.int64, device="cuda")
        pk.reshape_and_cache_fp8(rows_k, rows_v, kc, vc, slots, k_scale, v_scale)
    torch.cuda.synchronize()
    dev["k"], dev["v"] = kc, vc
    wl.k_cache = wl.v_cache = None
    dev.update(kv_fp8=True, k_scale=k_scale, v_scale=v_scale)


def grouped_lists(wl, dev, part_tiles=-1):
    """Inputs of the grouped decode call: sequences sharing their first block
    in groups of at most 16 / G (host set-up, not timed), the groups' tile
    lists from the host builder (for sizes; every timed step rebuilds them on
    the device with pkv_group_tiles), and the part size (-1: chosen from the
    list)."""
    from paged_kv_cache_389_amd import block_manager as bmod
    g = wl.num_q_heads // wl.num_kv_heads
    t0 = time.perf_counter()
    groups = bmod.share_groups(wl.block_tables, wl.context_lens, 16 // g)
    members, tiles, start = bmod.group_tiles(wl.block_tables, wl.context_lens, groups,
                                             wl.block_size, 16 // g)
    host_ms = (time.perf_counter() - t0) * 1e3
    if tiles.shape[0] == 0:
        tiles = np.zeros((1, 4), np.int32)
    max_group_tiles = int(np.diff(start).max(initial=0))
    if part_tiles < 0:
        # A full round of resident workgroups (4 per CU): the groups longer than
        # the mean are cut at the mean (rounded down to 16 tiles), so their tails
        # run as a second, short round instead of ending the launch alone
        # (sharing batch, 1024 workgroups: 0.2027-0.2069 ms with parts of 72-128
        # tiles against 0.2141 whole, the merge included in the call's 0.207).
        # Between one round and a quarter of one: whole groups (beam batch, 512
        # workgroups: parts of 16-96 tiles equal or up to 3% slower; system
        # prompt, 256: whole best).  Fewer: parts for about one round.
        wgs = len(groups) * wl.num_kv_heads
        lens = np.diff(start)
        if wgs >= 1024:
            part_tiles = max(16, 16 * int(lens.mean() // 16))
        elif wgs >= 256:
            part_tiles = 0
        else:
            part_tiles = max(8, -(-int(start[-1]) * wl.num_kv_heads // 1024))
    if dev is not None and torch.cuda.is_available():
        from paged_kv_cache_389_amd import _native as pk
        # the device builder's buffers: group j's rows from j * stride, start / end per group
        d_tiles, d_start, d_end = pk.group_tiles(
            torch.from_numpy(wl.block_tables).cuda(), torch.from_numpy(wl.context_lens).cuda(),
            torch.from_numpy(members).cuda(), wl.block_size, wl.max_context_len)
        dev["groups"] = (torch.from_numpy(members).cuda(), d_tiles, d_start)
        dev["group_end"] = d_end
        dev["group_part"] = (part_tiles, max_group_tiles)
        need = pk.grouped_workspace_bytes(len(groups), wl.num_kv_heads, wl.head_dim, part_tiles,
                                          max_group_tiles)
        dev["group_ws"] = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    return {"groups": len(groups), "max_members": 16 // g, "tiles": int(start[-1]),
            "part_tiles": part_tiles, "max_group_tiles": max_group_tiles,
            "logical_tiles": int(sum(-(-int(L) // 16) for L in wl.context_lens)),
            "host_list_ms": round(host_ms, 2)}


def grouped_decode_bytes(wl, info, kv_fp8=False):
    """What the grouped kernel must move: every distinct K/V tile once (one
    byte per element for 8-bit caches), q and out, its lists and the lengths."""
    return (wl.unique_kv_bytes() // (wl.esize if kv_fp8 else 1) + 2 * wl.num_seqs * wl.num_q_heads * wl.head_dim * wl.esize +
            16 * info["tiles"] + 4 * info["groups"] * info["max_members"] +
            4 * (info["groups"] + 1) + 4 * wl.num_seqs)


def run_gpu(wl, dev, steps, warmup, partition, path, grid):
    from paged_kv_cache_389_amd import _native as pk
    tables = None if (path & 0xFF) == 3 else dev["tables"]
    max_blocks = -(-wl.max_context_len // wl.block_size) if tables is None else tables.shape[1]
    fp8 = bool(dev.get("kv_fp8"))
    code = pk._DTYPE_CODE[wl.dtype] | (pk.KV_E4M3 if fp8 else 0)
    ws_len = pk.workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                wl.block_size, max_blocks, wl.max_context_len, code,
                                partition, path, grid)
    ws = torch.empty(max(ws_len, 1), dtype=torch.uint8, device="cuda")
    plan = pk.plan(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size,
                   max_blocks, wl.max_context_len, code, partition, path, grid)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    kev = [(pk.HipEvent(), pk.HipEvent()) for _ in range(steps)]

    def one_step(i=None, whole_call=False):
        if dev["pairs"] is not None:
            pk.copy_blocks(dev["k"], dev["v"], dev["pairs"])
        if dev["slots"] is not None:
            if fp8:
                pk.reshape_and_cache_fp8(dev["new_k"], dev["new_v"], dev["k"], dev["v"],
                                         dev["slots"], dev["k_scale"], dev["v_scale"])
            else:
                pk.reshape_and_cache(dev["new_k"], dev["new_v"], dev["k"], dev["v"],
                                     dev["slots"])
        if dev.get("groups") is not None:
            # the step's tile lists, built on the device from the block tables
            pk.group_tiles(dev["tables"], dev["lens"], dev["groups"][0], wl.block_size,
                           wl.max_context_len, tiles=dev["groups"][1],
                           tile_start=dev["groups"][2], tile_end=dev["group_end"])
        if whole_call:
            ev[i][0].record()
        if dev.get("groups") is not None:
            pk.paged_attention_decode_grouped(dev["out"], dev["q"], dev["k"], dev["v"],
                                              dev["lens"], *dev["groups"], wl.scale,
                                              wl.max_context_len,
                                              part_tiles=dev["group_part"][0],
                                              max_group_tiles=dev["group_part"][1],
                                              workspace=dev["group_ws"],
                                              group_tile_end=dev["group_end"],
                                              kernel_events=None if i is None or whole_call
                                              else kev[i],
                                              **({"k_scale": dev["k_scale"],
                                                  "v_scale": dev["v_scale"]} if fp8 else {}))
        elif fp8:
            pk.paged_attention_decode_fp8(dev["out"], dev["q"], dev["k"], dev["v"], tables,
                                          dev["lens"], wl.scale, dev["k_scale"], dev["v_scale"],
                                          wl.max_context_len, workspace=ws,
                                          partition_tokens=partition, path=path, grid=grid,
                                          kernel_events=None if i is None or whole_call
                                          else kev[i])
        else:
            pk.paged_attention_decode(dev["out"], dev["q"], dev["k"], dev["v"], tables,
                                      dev["lens"], wl.scale, wl.max_context_len, workspace=ws,
                                      partition_tokens=partition, path=path, grid=grid,
                                      kernel_events=None if i is None or whole_call else kev[i])
        if whole_call:
            ev[i][1].record()

    for _ in range(warmup):
        one_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        one_step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = [a.elapsed_ms(b) for a, b in kev]
    # the whole decode call, timed in a second pass outside the timed region so
    # that its event markers do not lengthen the timed steps
    for i in range(steps):
        one_step(i, whole_call=True)
    torch.cuda.synchronize()
    decode_ms = [a.elapsed_time(b) for a, b in ev]
    return wall, decode_ms, kernel_ms, plan


def bench_swap(args):
    """swap_blocks between the device cache and a pool in pinned host memory.

    Blocks of the llama-3-8B decode shape (8 KV heads x 16 tokens x 128,
    bf16: 32 KiB per K block and as much per V block); ``--swap`` pairs of
    distinct, randomly placed blocks go out (device -> host) and back in
    (host -> device) each step.  Throughput is K+V bytes moved over the
    kernel's time (torch events around the launch on the current stream),
    set against the host link's published peak (PCIe 5.0 x16, 64 GB/s per
    direction) and against a DMA copy of one contiguous buffer of the same
    size."""
    from paged_kv_cache_389_amd import _native as pk
    n = args.swap
    hkv, bs, hd, dt = 8, 16, 128, torch.bfloat16
    g = torch.Generator().manual_seed(389)
    dev_blocks, host_blocks = max(2 * n, 4096), n + n // 4
    kd = torch.randn((dev_blocks, hkv, bs, hd), generator=g).to(dt).cuda()
    vd = torch.randn((dev_blocks, hkv, bs, hd), generator=g).to(dt).cuda()
    kh = torch.zeros((host_blocks, hkv, bs, hd), dtype=dt).pin_memory()
    vh = torch.zeros((host_blocks, hkv, bs, hd), dtype=dt).pin_memory()
    d_sel = torch.randperm(dev_blocks, generator=g)[:n]
    h_sel = torch.randperm(host_blocks, generator=g)[:n]
    out_pairs = torch.stack([d_sel, h_sel], 1).cuda()
    in_pairs = torch.stack([h_sel, torch.randperm(dev_blocks, generator=g)[:n]], 1).cuda()
    moved = 2 * n * hkv * bs * hd * 2
    flat_d = torch.empty(moved, dtype=torch.uint8, device="cuda")
    flat_h = torch.empty(moved, dtype=torch.uint8).pin_memory()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev]))

    ms_out = timed(lambda: pk.swap_blocks(kd, vd, kh, vh, out_pairs))
    ms_in = timed(lambda: pk.swap_blocks(kh, vh, kd, vd, in_pairs))
    ms_dma_out = timed(lambda: flat_h.copy_(flat_d, non_blocking=True))
    ms_dma_in = timed(lambda: flat_d.copy_(flat_h, non_blocking=True))
    gbs = lambda ms: round(moved / (ms / 1e3) / 1e9, 2)
    both = 2 * moved / ((ms_out + ms_in) / 1e3) / 1e9
    print(json.dumps({
        "metric": "swap_blocks: K+V bytes moved per second, device <-> pinned host",
        "value": round(both, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_out + ms_in, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) values, random distinct block pairs)",
        "config": {"workload": "swap_llama3_8b_blocks", "pairs": n, "num_kv_heads": hkv,
                   "block_size": bs, "head_dim": hd, "bytes_each_way": moved},
        "out_gbs": gbs(ms_out), "in_gbs": gbs(ms_in),
        "dma_contiguous_out_gbs": gbs(ms_dma_out), "dma_contiguous_in_gbs": gbs(ms_dma_in),
        "roofline": {"bound": "host-link", "achieved": round(both, 2), "peak": HOST_LINK_GBS,
                     "unit": "GB/s", "frac": round(both / HOST_LINK_GBS, 4), "traffic": None,
                     "kernel": "copy_blocks_kernel"}}), flush=True)


def _oracle_inputs(wl, seqs):
    """The oracle's inputs for a set of sequences as host numpy arrays (the
    blocks they reference, compacted, in a type that holds the workload's
    values exactly: float16 stays float16, bfloat16 becomes float32)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_helpers import compact_pool
    kc, vc, tables = compact_pool(wl, seqs)
    host = (lambda t: t.numpy()) if wl.dtype != torch.bfloat16 else \
        (lambda t: t.float().numpy())
    return host(wl.q.cpu()), host(kc), host(vc), tables


def _time_oracle(q, kc, vc, tables, lens, scale, hkv, seqs, row, budget_s, rows_out=None):
    """Single-threaded oracle over ``seqs`` in order until ``budget_s``;
    returns (sequences done, KV bytes, seconds).  ``rows_out`` (a dict), if
    given, receives each sequence's oracle rows."""
    import oracle
    from threadpoolctl import threadpool_limits
    done, secs, kv = 0, 0.0, 0
    with threadpool_limits(limits=1):
        torch.set_num_threads(1)
        for s in seqs:
            t = time.perf_counter()
            o = oracle.decode(q, kc, vc, tables, lens, scale, hkv, seqs=[s])
            secs += time.perf_counter() - t
            if rows_out is not None:
                rows_out[s] = o[s]
            done += 1
            kv += int(lens[s]) * row
            if secs >= budget_s:
                break
    return done, kv, secs


def _pool_worker(path):
    """One process of the pooled CPU baseline: load its share (untimed),
    then time the oracle over it."""
    z = np.load(path)
    return _time_oracle(z["q"], z["kc"], z["vc"], z["tables"], z["lens"], float(z["scale"]),
                        int(z["hkv"]), [int(x) for x in z["seqs"]], int(z["row"]), float("inf"))


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 matrix peak


PREFILL_WARMUP = 100   # untimed prefill steps at least (see bench_prefill)


def bench_prefill(name, args, err_sample=None):
    """Causal prefill attention over the paged cache (every prompt token a
    query).  Throughput in causal attention TFLOP/s (4 * hd flops per query
    row, head and visible token) over the kernel's time (HIP events the
    library records around its launch), against the dense 16-bit MFMA peak;
    the minimum bytes (every K/V row once, q, out) give the HBM side.  With
    ``err_sample`` (16-bit pools), the first and last query rows of that many
    sequences (spread over the lengths) against the float64 oracle."""
    from paged_kv_cache_389_amd import _native as pk
    from paged_kv_cache_389_amd import workloads
    wl = workloads.make(name, device="cuda")
    tables = torch.from_numpy(wl.block_tables).cuda()
    lens = torch.from_numpy(wl.context_lens).cuda()
    qs = torch.from_numpy(wl.query_start).cuda()
    out = torch.empty_like(wl.q)
    kev = [(pk.HipEvent(), pk.HipEvent()) for _ in range(args.steps)]
    kv_bytes = int(wl.context_lens.astype(np.int64).sum()) * 2 * wl.num_kv_heads * wl.head_dim
    dev = {"k": wl.k_cache, "v": wl.v_cache}
    scales = {}
    if args.kv_cache == "e4m3":
        quantise_pools(wl, dev)
        scales = dict(k_scale=dev["k_scale"], v_scale=dev["v_scale"])

    def step(i=None):
        pk.paged_attention_prefill(out, wl.q, dev["k"], dev["v"], tables, lens, qs, wl.scale,
                                   wl.max_q_len, int(wl.context_lens.max()),
                                   kernel_events=None if i is None else kev[i], **scales)

    # A compute-bound kernel reaches the part's sustained clocks only after
    # some tens of milliseconds of work: with 3 warmup steps the timed ones
    # ran 0.417-0.421 ms, with 100 or 400 0.342-0.345 ms (the memory-bound
    # decode kernels move by 1% at most), so at least PREFILL_WARMUP steps.
    warmup = max(args.warmup, PREFILL_WARMUP)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = [a.elapsed_ms(b) for a, b in kev]
    ker = float(np.mean(kms))
    flops, nbytes = wl.flops(), wl.min_bytes()
    if dev.get("kv_fp8"):   # one byte per K/V element
        nbytes -= kv_bytes * (wl.esize - 1)
    tag = name + ("_kv_e4m3" if dev.get("kv_fp8") else "")
    tflops = flops / (ker / 1e3) / 1e12
    ms_per_step = wall / args.steps * 1e3
    err = {}
    if err_sample and not dev.get("kv_fp8"):
        err = prefill_oracle_error(wl, dev, out, err_sample)
    return {
        **err,
        "metric": "paged prefill attention: causal TFLOP/s (% of MFMA peak) + query tokens/s",
        "value": round(flops / (ms_per_step / 1e3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE_NAME[wl.dtype],
        "data": "synthetic (seeded N(0,1) values, random block placement)",
        "config": {"workload": tag, "kv_cache": "e4m3" if dev.get("kv_fp8") else
                   DTYPE_NAME[wl.dtype], "num_seqs": wl.num_seqs, "heads": f"{wl.num_q_heads}/"
                   f"{wl.num_kv_heads}", "head_dim": wl.head_dim, "block_size": wl.block_size,
                   "context_lens": "U[512,2048], every token a query", "total_q": wl.total_q,
                   "seed": wl.seed},
        "query_tokens_per_s": round(wl.total_q / (ms_per_step / 1e3), 1),
        "kernel_ms": round(ker, 5), "kernel_ms_median": round(float(np.median(kms)), 5),
        "kernel_ms_min": round(float(np.min(kms)), 5),
        "flops": flops, "min_bytes": nbytes,
        "hbm_gbs_at_min_bytes": round(nbytes / (ker / 1e3) / 1e9, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": recorded_traffic(tag), "kernel": "prefill_mfma_kernel"},
    }


def cpu_baseline(wl, budget_s, pool_workers=0, gpu_out=None):
    """The float64 oracle over whole sequences (all heads), throughput in the
    metric's unit (algorithmic KV GB/s of the sample).  One thread, in index
    order until the time budget is used; then, with ``pool_workers`` > 1, a
    process pool of that many single-threaded workers over the same number of
    sequences per worker (capped at the batch), each worker timing its own
    share after loading it: the pooled rate is the sample's bytes over the
    slowest worker's time."""
    row = 2 * wl.num_kv_heads * wl.head_dim * wl.esize
    order = list(range(wl.num_seqs))
    q, kc, vc, tables = _oracle_inputs(wl, order)
    rows = {}
    done, kv, secs = _time_oracle(q, kc, vc, tables, wl.context_lens, wl.scale,
                                  wl.num_kv_heads, order, row, budget_s, rows_out=rows)
    res = {"value": round(kv / secs / 1e9, 6), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "seconds": round(secs, 3), "queries_per_s": round(done / secs, 3),
           "sample": f"{done} of {wl.num_seqs} sequences x all {wl.num_q_heads} query heads "
                     f"(decode only, float64 numpy, one thread)"}
    if gpu_out is not None and rows:
        # the timed run's own output on the sampled sequences, against the oracle
        g = gpu_out.detach().to("cpu", torch.float64).numpy()
        res["max_abs_err_vs_gpu"] = float(max(np.abs(g[s] - r).max() for s, r in rows.items()))
    if pool_workers > 1:
        res["pool"] = _cpu_pool(wl, row, order[:min(wl.num_seqs, done * pool_workers)],
                                pool_workers)
    return res


def _cpu_pool(wl, row, seqs, workers):
    import concurrent.futures as cf
    import multiprocessing as mp
    import shutil
    import tempfile
    # longest first, dealt round-robin, so the workers' shares are alike
    seqs = sorted(seqs, key=lambda s: -int(wl.context_lens[s]))
    shares = [seqs[w::workers] for w in range(workers)]
    shares = [sh for sh in shares if sh]
    tmp = tempfile.mkdtemp(dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    try:
        paths = []
        for w, sh in enumerate(shares):
            path = os.path.join(tmp, f"share{w}.npz")
            q, kc, vc, tables = _oracle_inputs(wl, sh)   # only this share's blocks
            np.savez(path, q=q, kc=kc, vc=vc, tables=tables, lens=wl.context_lens,
                     scale=wl.scale, hkv=wl.num_kv_heads, seqs=np.array(sh), row=row)
            paths.append(path)
        with cf.ProcessPoolExecutor(len(paths), mp_context=mp.get_context("spawn")) as ex:
            results = list(ex.map(_pool_worker, paths))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    kv = sum(r[1] for r in results)
    slowest = max(r[2] for r in results)
    return {"value": round(kv / slowest / 1e9, 6), "unit": "GB/s", "cores": len(paths),
            "kind": "oracle", "seconds": round(slowest, 3),
            "queries_per_s": round(len(seqs) / slowest, 3),
            "sample": f"{len(seqs)} of {wl.num_seqs} sequences over {len(paths)} single-threaded "
                      f"worker processes (rate = sample bytes / slowest worker's oracle time)"}


def roofline_bytes(wl, kv_fp8=False, grouped=None, recorded_hbm=None):
    """Bytes the decode kernel's roofline fraction is taken on, and their
    basis.

    Every sequence's own K/V once (the algorithmic bytes) when no two
    sequences share a block; the grouped call's distinct tiles (each shared
    tile once) for the grouped kernel.  A per-sequence kernel over sequences
    that share blocks reads a shared block once per sequence, mostly from
    L2, so its logical bytes are not HBM bytes: there the basis is the
    counter-measured HBM bytes per launch when they were recorded for the
    current kernel sources, else the distinct slots' bytes (every shared
    slot once; a lower bound of the HBM bytes).  No basis exceeds the bytes
    the kernel moves from HBM, so the fraction stays at or below 1."""
    div = wl.esize if kv_fp8 else 1
    if grouped is not None:
        return grouped_decode_bytes(wl, grouped, kv_fp8), "unique K/V bytes (each distinct tile once)"
    logical = wl.decode_bytes() - (wl.kv_bytes() - wl.kv_bytes() // div)
    unique_kv = wl.unique_kv_bytes() // div
    if unique_kv >= wl.kv_bytes() // div:
        return logical, "algorithmic bytes (every sequence's own K/V once)"
    if recorded_hbm:
        return int(recorded_hbm), "counter-measured HBM bytes per launch (FETCH_SIZE + WRITE_SIZE)"
    return logical - wl.kv_bytes() // div + unique_kv, \
        "unique K/V bytes (each shared slot once: a lower bound of the HBM bytes)"


def _host_blocks(pool, blocks):
    """Host copies of the given physical blocks of a device pool, in a type
    that holds the values exactly (bfloat16 widened to float32)."""
    sel = torch.tensor(blocks, dtype=torch.int64, device=pool.device)
    t = pool.index_select(0, sel).cpu()
    return (t.float() if t.dtype == torch.bfloat16 else t).numpy()


def oracle_error(wl, dev, seqs, tables=None):
    """Max abs error of the timed run's output rows of ``seqs`` (all heads)
    against the float64 oracle over the same device pools (after the timed
    steps' cache writes).  ``tables`` overrides the block tables (the
    contiguous control reads block s * W + j)."""
    import oracle
    tables = wl.block_tables if tables is None else tables
    bs = wl.block_size
    used = sorted({int(b) for s in seqs for b in tables[s, :-(-int(wl.context_lens[s]) // bs)]})
    index = {b: i for i, b in enumerate(used)}
    ct = np.zeros(tables.shape, np.int64)
    for s in seqs:
        n = -(-int(wl.context_lens[s]) // bs)
        ct[s, :n] = [index[int(b)] for b in tables[s, :n]]
    q = dev["q"].cpu()
    q = (q.float() if q.dtype == torch.bfloat16 else q).numpy()
    want = oracle.decode(q, _host_blocks(dev["k"], used), _host_blocks(dev["v"], used), ct,
                         wl.context_lens, wl.scale, wl.num_kv_heads, seqs=list(seqs))
    got = dev["out"].detach().to("cpu", torch.float64).numpy()
    return float(max(np.abs(got[s] - want[s]).max() for s in seqs))


def prefill_oracle_error(wl, dev, out, count):
    """Max abs error of the timed prefill's first and last query rows of
    ``count`` sequences (all heads) against the float64 oracle, which reads
    only those sequences' blocks of the device pools."""
    import oracle
    seqs = oracle_sample(wl, count)
    bs = wl.block_size
    used = sorted({int(b) for s in seqs for b in wl.block_tables[s, :-(-int(wl.context_lens[s]) // bs)]})
    index = {b: i for i, b in enumerate(used)}
    ct = np.zeros(wl.block_tables.shape, np.int64)
    rows = []
    for s in seqs:
        n = -(-int(wl.context_lens[s]) // bs)
        ct[s, :n] = [index[int(b)] for b in wl.block_tables[s, :n]]
        q0, q1 = int(wl.query_start[s]), int(wl.query_start[s + 1])
        rows += sorted({q0, q1 - 1}) if q1 > q0 else []
    q = wl.q.cpu()
    q = (q.float() if q.dtype == torch.bfloat16 else q).numpy()
    want = oracle.prefill(q, _host_blocks(dev["k"], used), _host_blocks(dev["v"], used), ct,
                          wl.context_lens, wl.query_start, wl.scale, wl.num_kv_heads, rows=rows)
    got = out.detach().to("cpu", torch.float64).numpy()
    return {"max_abs_err": float(max(np.abs(got[r] - want[r]).max() for r in rows)),
            "tol": TOL[wl.dtype],
            "err_sample": f"first and last query rows of {len(seqs)} of {wl.num_seqs} sequences "
                          f"(all {wl.num_q_heads} heads) against the float64 oracle"}


def prefill_entry(line):
    """The prefill summary the default run reports beside the decode configs."""
    r = line["roofline"]
    return {"kernel": r["kernel"], "workload": line["config"]["workload"],
            "kernel_ms": line["kernel_ms"], "kernel_ms_median": line["kernel_ms_median"],
            "flops": line["flops"], "achieved_tflops": r["achieved"], "peak_tflops": r["peak"],
            "frac": r["frac"], "traffic": r["traffic"], "min_bytes": line["min_bytes"],
            "query_tokens_per_s": line["query_tokens_per_s"], "warmup": line["warmup"],
            "max_abs_err": line.get("max_abs_err"), "tol": line.get("tol"),
            "err_sample": line.get("err_sample")}


def oracle_sample(wl, count):
    """``count`` sequences spread evenly over the batch sorted by length
    (the longest and the shortest included)."""
    order = np.argsort(-wl.context_lens.astype(np.int64), kind="stable")
    if count >= len(order):
        return sorted(int(s) for s in order)
    pick = np.unique(np.rint(np.linspace(0, len(order) - 1, count)).astype(int))
    return sorted(int(order[i]) for i in pick)


ERR_SAMPLE = {"tiny_fp32": 4, "opt13b_fp16": 8, "llama3_8b_gqa_bf16": 16,
              "long_context_gqa_bf16": 2, "sharing_fp16": 8, "beam_search_fp16": 8,
              "system_prompt_bf16": 8}
TOL = {torch.float32: 1e-5, torch.float16: 2e-2, torch.bfloat16: 2e-2}


def bench_one(name, args, with_cpu, placement=None, path=None, err_sample=None):
    placement = args.placement if placement is None else placement
    path = args.path if path is None else path
    wl, dev = build_inputs(name, placement)
    if args.kv_cache == "e4m3":
        with_cpu = False   # the oracle baseline times the 16-bit pools
        quantise_pools(wl, dev)
    fp8 = bool(dev.get("kv_fp8"))
    grouped = None
    if args.grouped:
        grouped = grouped_lists(wl, dev, args.group_part)
    tag = name + ("_kv_e4m3" if fp8 else "") + ("_grouped" if grouped else "")
    _, alg_writes = step_bytes(wl, dev)
    recorded = recorded_traffic(tag)
    alg_decode, basis = roofline_bytes(wl, fp8, grouped, recorded)
    # the caller knows when its sequences share blocks: the per-sequence
    # decode then keeps K/V in the cache for the other holders of a block
    shared = name in GROUPABLE and not grouped
    call_path = path | (0x100 if shared else 0)
    wall, decode_ms, kernel_ms, plan = run_gpu(wl, dev, args.steps, args.warmup, args.partition,
                                               call_path, args.grid)
    ms_per_step = wall / args.steps * 1e3
    dec_ms = float(np.mean(decode_ms))
    ker_ms = float(np.mean(kernel_ms))
    achieved = alg_decode / (ker_ms / 1e3) / 1e9
    kname = ("decode_grouped_kernel" if grouped else
             "decode_mfma_kernel" if plan["path"] == 2 else "decode_valu_kernel")
    logical = wl.kv_bytes() // (wl.esize if fp8 else 1)
    line = {
        "metric": "paged decode attention: achieved KV HBM GB/s (% of peak) + queries/s",
        "value": round((alg_decode + alg_writes) / (ms_per_step / 1e3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[wl.dtype],
        "data": "synthetic (seeded N(0,1) values, "
                f"{'random' if placement == 'random' else 'sequential'} block placement)",
        "config": {"workload": tag,
                   **WORKLOAD_DESC[name], "seed": wl.seed,
                   "kv_cache": "e4m3" if fp8 else DTYPE_NAME[wl.dtype],
                   "placement": placement,
                   "path": ["auto", "valu", "mfma", "contiguous"][path],
                   "kv_loads": "cached (blocks shared across the batch)" if shared
                   else "streaming (nontemporal)",
                   "kernel": ["auto", "valu", "mfma"][plan["path"]],
                   "grid": {1: "direct", 2: "planned"}[plan["grid"]],
                   "partition_tokens": plan["partition_tokens"], "max_parts": plan["max_parts"],
                   "longest_first": bool(plan["longest_first"])},
        "queries_per_s": round(wl.num_seqs / (ms_per_step / 1e3), 1),
        "kv_utilisation": round(float(wl.meta["utilisation"]), 4) if "utilisation" in wl.meta
        else None,
        "pct_of_hbm_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
        "decode_ms": round(dec_ms, 5),
        "decode_ms_min": round(float(np.min(decode_ms)), 5),
        "kernel_ms": round(ker_ms, 5),
        "kernel_ms_median": round(float(np.median(kernel_ms)), 5),
        "kernel_ms_min": round(float(np.min(kernel_ms)), 5),
        "gbs_at_median": round(alg_decode / (float(np.median(kernel_ms)) / 1e3) / 1e9, 2),
        "bytes": {"decode_roofline": alg_decode, "writes_alg": alg_writes,
                  "kv_logical": logical},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded, "kernel": kname, "basis": basis},
    }
    if grouped:
        for k in ("partition_tokens", "max_parts", "longest_first"):   # the per-sequence plan's
            line["config"].pop(k, None)
        line["config"]["kernel"] = "grouped"
        line["config"]["grid"] = "groups x kv heads x parts"
        line["config"]["part_tiles"] = grouped["part_tiles"]
        line["config"]["lists"] = "built on the device every step (group_tiles, timed)"
        line["grouped"] = grouped
    unique = wl.unique_kv_bytes() // (wl.esize if fp8 else 1)
    if unique < logical:
        line["bytes"]["kv_unique"] = unique
        line["logical_kv_gbs"] = round(logical / (ker_ms / 1e3) / 1e9, 2)
        line["sharing_saving"] = round(1.0 - unique / logical, 4)
    if name == "system_prompt_bf16":
        bs = wl.block_size
        logical_blocks = int(((wl.context_lens.astype(np.int64) + bs - 1) // bs).sum())
        line["system_prompt"] = {
            "copy_pairs_admission": int(len(wl.history[0].copy_pairs)),
            "block_saving_vs_unshared": round(
                1.0 - (wl.meta["physical_blocks"] - sum(len(t) for t in wl.meta["entry_tables"]))
                / logical_blocks, 4)}
    if name == "beam_search_fp16":
        from paged_kv_cache_389_amd import workloads
        pairs = [len(h.copy_pairs) for h in wl.history]
        line["beam"] = {"copy_pairs_timed_step": pairs[-1],
                        "copy_pairs_per_step_mean": round(float(np.mean(pairs)), 2),
                        "block_saving_vs_unshared": round(workloads.sharing_saving(wl), 4)}
    if err_sample and not fp8:
        seqs = oracle_sample(wl, err_sample)
        tables = None
        if path == 3:   # the contiguous control reads block s * W + j
            w = -(-wl.max_context_len // wl.block_size)
            tables = (np.arange(wl.num_seqs)[:, None] * w + np.arange(w)[None, :]).astype(np.int64)
        line["max_abs_err"] = oracle_error(wl, dev, seqs, tables)
        line["tol"] = TOL[wl.dtype]
        line["err_sample"] = f"{len(seqs)} of {wl.num_seqs} sequences (longest and shortest " \
                             f"included), all {wl.num_q_heads} heads, vs the float64 oracle"
    if with_cpu:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget_s, args.cpu_pool, dev["out"])
    del wl, dev
    return line


def config_entry(line):
    """The per-configuration summary of one bench line."""
    r = line["roofline"]
    e = {"kernel": r["kernel"], "plan": {k: line["config"][k] for k in
                                         ("grid", "partition_tokens", "max_parts", "part_tiles")
                                         if k in line["config"]},
         "kernel_ms": line["kernel_ms"], "decode_ms": line["decode_ms"],
         "step_ms": line["ms_per_step"], "roofline_bytes": line["bytes"]["decode_roofline"],
         "basis": r["basis"], "achieved_gbs": r["achieved"], "frac": r["frac"],
         "traffic": r["traffic"], "queries_per_s": line["queries_per_s"],
         "max_abs_err": line.get("max_abs_err"), "tol": line.get("tol"),
         "err_sample": line.get("err_sample")}
    if line["bytes"]["writes_alg"]:
        e["step_bytes_writes"] = line["bytes"]["writes_alg"]
    for k in ("logical_kv_gbs", "sharing_saving"):
        if k in line:
            e[k] = line[k]
    return e


# the configurations every default run reports, beside the headline
PER_CONFIG = (("tiny_fp32", "tiny_fp32", False),
              ("llama3_8b_gqa_bf16", "llama3_8b_gqa_bf16", False),
              ("long_context_gqa_bf16", "long_context_gqa_bf16", False),
              ("sharing_fp16", "sharing_fp16", False),
              ("sharing_fp16_grouped", "sharing_fp16", True),
              # next rows: requests sharing cached system prompts, both decodes
              ("system_prompt_bf16", "system_prompt_bf16", False),
              ("system_prompt_bf16_grouped", "system_prompt_bf16", True))


def per_config(args, headline):
    """Summaries of every configuration (the headline's included) and the
    full lines they come from."""
    out, lines = {"opt13b_fp16": config_entry(headline)}, {}
    grouped0 = args.grouped
    for key, name, grouped in PER_CONFIG:
        args.grouped = grouped
        lines[key] = bench_one(name, args, False, err_sample=ERR_SAMPLE[name])
        out[key] = config_entry(lines[key])
    args.grouped = grouped0
    return out, lines


def paging_control(args, headline=None, long_line=None, rounds=3):
    """The block-table overhead control: the same kernels with random
    placement (the workload), sequential placement (blocks in increasing
    physical order) and no table at all (block j of sequence s at s * W +
    j), on the OPT-13B-shaped and the long-context batches.  The three run
    in turn, ``rounds`` times (a run's median differs by a few percent from
    one run to the next); each variant reports the median of its runs'
    median kernel times, and its first run's error against the oracle."""
    res = {}
    variants = (("random", {}), ("sequential", {"placement": "sequential"}),
                ("contiguous", {"path": 3}))
    for name, base in (("opt13b_fp16", headline), ("long_context_gqa_bf16", long_line)):
        runs = {k: [] for k, _ in variants}
        if base is not None:
            runs["random"].append(base)
        for r in range(rounds):
            for k, kw in variants:
                if len(runs[k]) > r:
                    continue
                runs[k].append(bench_one(name, args, False, err_sample=ERR_SAMPLE[name]
                                         if r == 0 else None, **kw))
        ent = {}
        for k, lines in runs.items():
            meds = [ln["kernel_ms_median"] for ln in lines]
            ent[k] = {"kernel_ms_median": round(float(np.median(meds)), 5),
                      "kernel_ms_medians": meds,
                      "frac": round(float(np.median([ln["roofline"]["frac"] for ln in lines])), 4),
                      "max_abs_err": lines[0].get("max_abs_err")}
        r = ent["random"]["kernel_ms_median"]
        ent["random_over_sequential"] = round(r / ent["sequential"]["kernel_ms_median"], 4)
        ent["random_over_contiguous"] = round(r / ent["contiguous"]["kernel_ms_median"], 4)
        res[name] = ent
    return res


def practical_ceiling(reps=10):
    """Reference reads (``csrc/ceiling.hip``): a contiguous 2 GiB stream, and a
    gather of random distinct 4 KiB and 8 KiB chunks (one 16-token tile of a
    16-bit hd-128 cache; a 32-token one) from a 2 GiB pool with streaming
    loads; then 4 KiB chunks with cached loads, and the K and V chunks of one
    index from two 1 GiB pools (streaming and cached); each at a few grid
    sizes, GB/s of the best, from torch events around each launch."""
    from paged_kv_cache_389_amd import _native as pk
    nbytes = 2 << 30
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").random_()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cpu").manual_seed(389)
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def best(fn, moved, grids):
        out = {}
        for wgs in grids:
            for _ in range(3):
                fn(wgs)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(reps)]
            for a, b in ev:
                a.record()
                fn(wgs)
                b.record()
            torch.cuda.synchronize()
            ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
            out[wgs] = round(moved / (ms / 1e3) / 1e9, 1)
        return max(out.values()), out

    res = {"peak_gbs": HBM_PEAK_GBS}
    s_best, s_all = best(lambda w: pk.ceiling_stream_read(buf, w, sink), nbytes,
                         [cus * k for k in (2, 4, 8, 16)])
    res["stream_read_gbs"] = s_best
    res["stream_read_by_workgroups"] = s_all
    for cb in (4096, 8192):
        n = (3 * nbytes // 4) // cb    # three quarters of the pool, random distinct chunks
        chunks = torch.randperm(nbytes // cb, generator=g)[:n].to(torch.int32).cuda()
        moved = n * cb
        g_best, g_all = best(lambda w: pk.ceiling_gather_read(buf, chunks, cb, w, sink), moved,
                             [cus * k for k in (2, 4, 8)])
        res[f"gather_{cb // 1024}k_gbs"] = g_best
        res[f"gather_{cb // 1024}k_by_workgroups"] = g_all
    # 4 KiB chunks with the cache's default policy, and the K and V tiles of one
    # index from two pools (the decode's pattern), streaming and cached
    half = buf.numel() // 2
    k_pool, v_pool = buf[:half], buf[half:]
    n = (3 * (nbytes // 2) // 4) // 4096
    chunks = torch.randperm((nbytes // 2) // 4096, generator=g)[:n].to(torch.int32).cuda()
    variants = (("gather_4k_cached", buf, None, True, (3 * nbytes // 4) // 4096),
                ("gather_4k_two_pools", k_pool, v_pool, False, n),
                ("gather_4k_two_pools_cached", k_pool, v_pool, True, n))
    for name, p1, p2, cached, cnt in variants:
        ch = chunks if p2 is not None else torch.randperm(nbytes // 4096, generator=g)[:cnt].to(
            torch.int32).cuda()
        moved = cnt * 4096 * (2 if p2 is not None else 1)
        g_best, g_all = best(lambda w: pk.ceiling_gather_read(p1, ch, 4096, w, sink, pool2=p2,
                                                              cached=cached), moved,
                             [cus * k for k in (2, 4)])
        res[name + "_gbs"] = g_best
        res[name + "_by_workgroups"] = g_all
    res["frac_of_peak"] = {k: round(v / HBM_PEAK_GBS, 4) for k, v in res.items()
                           if k.endswith("_gbs") and k != "peak_gbs"}
    del buf
    return res


def main():
    args = parse()
    if args.counters:
        counters_to_traffic(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path needs no communication; see the sharding notes)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.swap:
        bench_swap(args)
        return
    if args.ceiling:
        print(json.dumps({"practical_ceiling": practical_ceiling()}), flush=True)
        return
    if args.workload in PREFILL_WORKLOADS:
        print(json.dumps(bench_prefill(args.workload, args)), flush=True)
        return
    if args.sweep:
        for name in sorted(WORKLOAD_DESC):
            line = bench_one(name, args, with_cpu=False, err_sample=ERR_SAMPLE.get(name))
            print(json.dumps(line), flush=True)
            if not args.grouped and name in GROUPABLE:
                args.grouped = True    # the same batch through the grouped call
                print(json.dumps(bench_one(name, args, with_cpu=False,
                                           err_sample=ERR_SAMPLE.get(name))), flush=True)
                args.grouped = False
        return
    line = bench_one(args.workload, args, with_cpu=not args.no_cpu_baseline,
                     err_sample=ERR_SAMPLE.get(args.workload))
    full = (args.workload == DEFAULT_WORKLOAD and not args.quick and not args.grouped and
            args.kv_cache == "auto" and args.placement == "random" and args.path == 0 and
            args.partition == 0 and args.grid == 0)
    if full:
        t0 = time.perf_counter()
        line["per_config"], lines = per_config(args, line)
        # the next row's causal prefill, on the matrix-core roofline
        line["prefill"] = prefill_entry(bench_prefill("llama3_8b_prefill_bf16", args, err_sample=4))
        line["paging_control"] = paging_control(args, line, lines.get("long_context_gqa_bf16"))
        line["practical_ceiling"] = practical_ceiling()
        line["extra_s"] = round(time.perf_counter() - t0, 1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
