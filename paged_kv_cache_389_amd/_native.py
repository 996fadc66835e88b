"""ctypes binding of libpagedkv.so (argument marshalling only).

Every function takes torch tensors that live on a HIP device, checks their
shapes and dtypes against the C contract (``include/pagedkv.h``), and passes
raw device pointers plus the current HIP stream to the C ABI.  All compute
runs in the library's kernels.  If the library is not built, importing this
module raises: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

import torch  # loads torch's HIP runtime first, so the library shares it

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

PKV_F32, PKV_F16, PKV_BF16, PKV_E4M3 = 0, 1, 2, 3
KV_E4M3 = 0x100   # OR-ed into a q dtype code: the caches hold E4M3 codes
PATH_AUTO, PATH_VALU, PATH_MFMA, PATH_CONTIGUOUS = 0, 1, 2, 3
# OR-ed into a path: the batch's sequences share blocks (cached K/V loads)
PATH_SHARED_BLOCKS = 0x100
_DTYPE_CODE = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16}
# element types of caches the byte-moving calls accept (uint8: E4M3 codes)
_CACHE_CODE = {**_DTYPE_CODE, torch.uint8: PKV_E4M3}
_SIZE_MAX = ctypes.c_size_t(-1).value


GRID_AUTO, GRID_DIRECT, GRID_PLANNED = 0, 1, 2


class _Plan(ctypes.Structure):
    """Mirror of ``pkv_plan`` in include/pagedkv.h."""
    _fields_ = [("path", ctypes.c_int), ("grid", ctypes.c_int),
                ("partition_tokens", ctypes.c_int), ("max_parts", ctypes.c_int),
                ("longest_first", ctypes.c_int), ("workspace_bytes", ctypes.c_size_t)]


class NativeLibraryMissing(ImportError):
    pass


class PagedKVError(RuntimeError):
    def __init__(self, call, status, lib):
        msg = lib.pkv_status_string(status).decode()
        detail = lib.pkv_last_error().decode()
        super().__init__(f"{call} failed: {msg} ({status})" + (f": {detail}" if detail else ""))
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise NativeLibraryMissing(
            f"{LIB_PATH} is missing; build it with `python -m paged_kv_cache_389_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64p, i32p = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p
    f32, sz = ctypes.c_float, ctypes.c_size_t
    lib.pkv_version.restype = ctypes.c_char_p
    lib.pkv_version.argtypes = []
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_status_string.argtypes = [i32]
    lib.pkv_last_error.restype = ctypes.c_char_p
    lib.pkv_last_error.argtypes = []
    lib.pkv_supported.restype = i32
    lib.pkv_supported.argtypes = [i32, i32, i32]
    lib.pkv_paged_attention_workspace_bytes.restype = sz
    lib.pkv_paged_attention_workspace_bytes.argtypes = [i32] * 11
    lib.pkv_paged_attention_plan.restype = i32
    lib.pkv_paged_attention_plan.argtypes = [i32] * 11 + [ctypes.POINTER(_Plan)]
    lib.pkv_paged_attention_decode.restype = i32
    lib.pkv_paged_attention_decode.argtypes = [
        vp, vp, vp, vp, i32p, i32p, f32, i32, i32, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    lib.pkv_paged_attention_decode_ex.restype = i32
    lib.pkv_paged_attention_decode_ex.argtypes = [
        vp, vp, vp, vp, i32p, i32p, f32, i32, i32, i32, i32, i32, i32, i32, i32, i32, vp, sz,
        i32, i32, i32, vp]
    lib.pkv_paged_attention_decode_timed.restype = i32
    lib.pkv_paged_attention_decode_timed.argtypes = [
        vp, vp, vp, vp, i32p, i32p, f32, i32, i32, i32, i32, i32, i32, i32, i32, i32, vp, sz,
        i32, i32, i32, vp, vp, vp]
    lib.pkv_reshape_and_cache.restype = i32
    lib.pkv_reshape_and_cache.argtypes = [vp, vp, vp, vp, i64p, i32, i32, i32, i32, i32, i32, vp]
    lib.pkv_copy_blocks.restype = i32
    lib.pkv_copy_blocks.argtypes = [vp, vp, i64p, i32, i32, i32, i32, i32, i32, vp]
    lib.pkv_swap_blocks.restype = i32
    lib.pkv_swap_blocks.argtypes = [vp, vp, vp, vp, i64p, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.pkv_reshape_and_cache_fp8.restype = i32
    lib.pkv_reshape_and_cache_fp8.argtypes = [vp, vp, vp, vp, i64p, i32, i32, i32, i32, i32, i32,
                                              f32, f32, vp]
    lib.pkv_paged_attention_decode_fp8.restype = i32
    lib.pkv_paged_attention_decode_fp8.argtypes = [
        vp, vp, vp, vp, i32p, i32p, f32, f32, f32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
        vp, sz, i32, i32, i32, vp, vp, vp]
    lib.pkv_paged_attention_prefill.restype = i32
    lib.pkv_paged_attention_prefill.argtypes = [
        vp, vp, vp, vp, i32p, i32p, i32p, f32, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
        i32, vp, vp, vp]
    lib.pkv_paged_attention_prefill_fp8.restype = i32
    lib.pkv_paged_attention_prefill_fp8.argtypes = [
        vp, vp, vp, vp, i32p, i32p, i32p, f32, f32, f32, i32, i32, i32, i32, i32, i32, i32, i32,
        i32, i32, i32, vp, vp, vp]
    lib.pkv_paged_attention_decode_grouped.restype = i32
    lib.pkv_paged_attention_decode_grouped.argtypes = [
        vp, vp, vp, vp, i32p, i32p, i32p, i32p, i32p, i32, f32, i32, i32, i32, i32, i32, i32,
        i32, i32, i32, i32, i32, i32, vp, sz, vp, vp, vp]
    lib.pkv_paged_attention_decode_grouped_fp8.restype = i32
    lib.pkv_paged_attention_decode_grouped_fp8.argtypes = [
        vp, vp, vp, vp, i32p, i32p, i32p, i32p, i32p, i32, f32, f32, f32, i32, i32, i32, i32,
        i32, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp, vp, vp]
    lib.pkv_group_tiles.restype = i32
    lib.pkv_group_tiles.argtypes = [i32p, i32p, i32p, i32, i32, i32, i32, i32, i32, i32p, i32,
                                    i32p, i32p, vp]
    lib.pkv_group_tiles_capacity.restype = sz
    lib.pkv_group_tiles_capacity.argtypes = [i32] * 5
    lib.pkv_paged_attention_grouped_workspace_bytes.restype = sz
    lib.pkv_paged_attention_grouped_workspace_bytes.argtypes = [i32] * 5
    lib.pkv_paged_attention_decode_noalloc.restype = i32
    lib.pkv_paged_attention_decode_noalloc.argtypes = [
        vp, vp, vp, vp, i32p, i32p, f32, i32, i32, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.pkv_ceiling_stream_read.restype = i32
    lib.pkv_ceiling_stream_read.argtypes = [vp, sz, i32, vp, vp]
    lib.pkv_ceiling_gather_read.restype = i32
    lib.pkv_ceiling_gather_read.argtypes = [vp, vp, sz, i32p, i32, i32, i32, i32, vp, vp]
    return lib


lib = _load()

EXPORTED = (
    "pkv_version", "pkv_status_string", "pkv_last_error", "pkv_supported",
    "pkv_paged_attention_workspace_bytes", "pkv_paged_attention_plan",
    "pkv_paged_attention_decode",
    "pkv_paged_attention_decode_ex", "pkv_paged_attention_decode_timed",
    "pkv_reshape_and_cache", "pkv_copy_blocks", "pkv_swap_blocks",
    "pkv_reshape_and_cache_fp8", "pkv_paged_attention_decode_fp8",
    "pkv_paged_attention_prefill", "pkv_paged_attention_prefill_fp8",
    "pkv_paged_attention_decode_grouped", "pkv_paged_attention_decode_grouped_fp8",
    "pkv_paged_attention_grouped_workspace_bytes", "pkv_group_tiles", "pkv_group_tiles_capacity",
    "pkv_ceiling_stream_read", "pkv_ceiling_gather_read", "pkv_paged_attention_decode_noalloc",
)
NOALLOC_SCRATCH_BYTES = 32 << 20   # PKV_NOALLOC_SCRATCH_BYTES


def version() -> str:
    return lib.pkv_version().decode()


def _check(call, status):
    if status != 0:
        raise PagedKVError(call, status, lib)


def _dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(t: torch.Tensor, stream):
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _dtype_code(dtype):
    if isinstance(dtype, int):
        return dtype
    if dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {dtype}")
    return _DTYPE_CODE[dtype]


def plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
         max_context_len, dtype, partition_tokens=0, path=PATH_AUTO, grid=GRID_AUTO):
    """The plan of a decode call with these sizes, as a dict with the fields
    of ``pkv_plan``: path, grid, partition_tokens, max_parts, longest_first,
    workspace_bytes (see ``pkv_paged_attention_plan``)."""
    out = _Plan()
    st = lib.pkv_paged_attention_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                      max_blocks_per_seq, max_context_len, _dtype_code(dtype),
                                      partition_tokens, path, grid, ctypes.byref(out))
    _check("paged_attention_plan", st)
    return {name: getattr(out, name) for name, _ in _Plan._fields_}


def workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                    max_blocks_per_seq, max_context_len, dtype, partition_tokens=0,
                    path=PATH_AUTO, grid=GRID_AUTO) -> int:
    n = lib.pkv_paged_attention_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                block_size, max_blocks_per_seq, max_context_len,
                                                _dtype_code(dtype), partition_tokens, path, grid)
    if n == _SIZE_MAX:
        raise ValueError("invalid sizes for the decode workspace")
    return int(n)


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                           max_context_len, workspace=None, partition_tokens=0,
                           path=PATH_AUTO, grid=GRID_AUTO, stream=None, kernel_events=None):
    """``out[s, h] = softmax(scale * K_s q[s, h]) V_s`` over each sequence's
    paged KV (see ``pkv_paged_attention_decode``).  ``max_context_len`` is a
    host-side bound of ``context_lens``.  ``workspace`` is a uint8 device
    tensor; when None one of the required size is allocated.
    ``kernel_events`` = (begin, end) :class:`HipEvent` pair recorded around
    the attention kernel itself (``pkv_paged_attention_decode_timed``)."""
    for t, n in ((out, "out"), (q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                 (context_lens, "context_lens")):
        _dev(t, n)
    if (path & 0xFF) != PATH_CONTIGUOUS or block_tables is not None:
        _dev(block_tables, "block_tables")
        if block_tables.dtype != torch.int32 or block_tables.dim() != 2:
            raise ValueError("block_tables must be int32 [num_seqs, max_blocks]")
    if q.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for t, n in ((out, "out"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        if t.dtype != q.dtype:
            raise ValueError(f"{n} dtype {t.dtype} != q dtype {q.dtype}")
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must both be [num_seqs, num_q_heads, head_dim]")
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("caches must both be [num_blocks, num_kv_heads, block_size, head_dim]")
    num_seqs, hq, hd = q.shape
    nb, hkv, bs, hd2 = k_cache.shape
    if hd2 != hd:
        raise ValueError("head_dim of q and caches differ")
    if context_lens.dtype != torch.int32 or context_lens.shape != (num_seqs,):
        raise ValueError("context_lens must be int32 [num_seqs]")
    max_blocks = block_tables.shape[1] if block_tables is not None else \
        -(-int(max_context_len) // bs)
    if block_tables is not None and block_tables.shape[0] != num_seqs:
        raise ValueError("block_tables must have num_seqs rows")
    need = workspace_bytes(num_seqs, hq, hkv, hd, bs, max_blocks, int(max_context_len), q.dtype,
                           partition_tokens, path, grid)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    tables_ptr = _ptr(block_tables) if block_tables is not None else None
    with torch.cuda.device(q.device):
        ev0, ev1 = (kernel_events[0].handle, kernel_events[1].handle) if kernel_events \
            else (None, None)
        st = lib.pkv_paged_attention_decode_timed(
            _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), tables_ptr, _ptr(context_lens),
            ctypes.c_float(scale), num_seqs, hq, hkv, hd, bs, nb, max_blocks,
            int(max_context_len), _DTYPE_CODE[q.dtype], ws_ptr, ws_len, int(partition_tokens),
            int(path), int(grid), ev0, ev1, _stream(q, stream))
    _check("paged_attention_decode", st)
    return out


def paged_attention_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                   max_context_len, stream=None):
    """:func:`paged_attention_decode` without a workspace argument: the
    library's own device scratch serves as workspace
    (``pkv_paged_attention_decode_noalloc``), so nothing is allocated; calls
    whose plan needs more than ``NOALLOC_SCRATCH_BYTES`` raise.  Calls on one
    device share that scratch and must be ordered (one stream)."""
    for t, n in ((out, "out"), (q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                 (block_tables, "block_tables"), (context_lens, "context_lens")):
        _dev(t, n)
    if q.dtype not in _DTYPE_CODE or any(t.dtype != q.dtype for t in (out, k_cache, v_cache)):
        raise ValueError("q, out and both caches must share one supported dtype")
    if q.dim() != 3 or out.shape != q.shape or k_cache.dim() != 4 or \
            v_cache.shape != k_cache.shape or k_cache.shape[3] != q.shape[2]:
        raise ValueError("q/out [num_seqs, Hq, hd] and caches [num_blocks, Hkv, bs, hd] expected")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or \
            context_lens.dtype != torch.int32 or context_lens.shape != (q.shape[0],) or \
            block_tables.shape[0] != q.shape[0]:
        raise ValueError("block_tables int32 [num_seqs, W] and context_lens int32 [num_seqs]")
    num_seqs, hq, hd = q.shape
    nb, hkv, bs, _ = k_cache.shape
    with torch.cuda.device(q.device):
        st = lib.pkv_paged_attention_decode_noalloc(
            _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            _ptr(context_lens), ctypes.c_float(scale), num_seqs, hq, hkv, hd, bs, nb,
            block_tables.shape[1], int(max_context_len), _DTYPE_CODE[q.dtype],
            _stream(q, stream))
    _check("paged_attention_decode_noalloc", st)
    return out


def reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, stream=None):
    """Write new tokens' K/V rows ([num_tokens, Hkv, hd]) into the cache slots
    ``slot_mapping`` (int64, negative = skip)."""
    for t, n in ((k, "k"), (v, "v"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                 (slot_mapping, "slot_mapping")):
        _dev(t, n)
    if k.dtype not in _DTYPE_CODE or any(t.dtype != k.dtype for t in (v, k_cache, v_cache)):
        raise ValueError("k, v and both caches must share one supported dtype")
    if k.dim() != 3 or v.shape != k.shape:
        raise ValueError("k and v must both be [num_tokens, num_kv_heads, head_dim]")
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("caches must both be [num_blocks, num_kv_heads, block_size, head_dim]")
    nb, hkv, bs, hd = k_cache.shape
    if k.shape[1:] != (hkv, hd):
        raise ValueError("k/v rows do not match the cache's [num_kv_heads, head_dim]")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (k.shape[0],):
        raise ValueError("slot_mapping must be int64 [num_tokens]")
    with torch.cuda.device(k.device):
        st = lib.pkv_reshape_and_cache(_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(slot_mapping), k.shape[0], hkv, hd, bs, nb,
                                       _DTYPE_CODE[k.dtype], _stream(k, stream))
    _check("reshape_and_cache", st)


def copy_blocks(k_cache, v_cache, src_dst_pairs, stream=None):
    """Copy whole blocks ``cache[dst] = cache[src]`` for each int64 pair row."""
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"), (src_dst_pairs, "src_dst_pairs")):
        _dev(t, n)
    if k_cache.dtype not in _CACHE_CODE or v_cache.dtype != k_cache.dtype:
        raise ValueError("caches must share one supported dtype")
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("caches must both be [num_blocks, num_kv_heads, block_size, head_dim]")
    if src_dst_pairs.dtype != torch.int64 or src_dst_pairs.dim() != 2 or \
            src_dst_pairs.shape[1] != 2:
        raise ValueError("src_dst_pairs must be int64 [num_pairs, 2]")
    nb, hkv, bs, hd = k_cache.shape
    with torch.cuda.device(k_cache.device):
        st = lib.pkv_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(src_dst_pairs),
                                 src_dst_pairs.shape[0], hkv, hd, bs, nb,
                                 _CACHE_CODE[k_cache.dtype], _stream(k_cache, stream))
    _check("copy_blocks", st)


def _reachable(t: torch.Tensor, name: str):
    """A tensor the device can address: HIP device memory or pinned host memory."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda" and not (t.device.type == "cpu" and t.is_pinned()):
        raise ValueError(f"{name} must be on a HIP device or in pinned host memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def swap_blocks(src_k, src_v, dst_k, dst_v, src_dst_pairs, stream=None):
    """``dst[pair[1]] = src[pair[0]]`` for whole blocks of the K and V pools,
    between the device cache and a pool in pinned host memory (either way;
    ``pkv_swap_blocks``).  ``src_dst_pairs`` is int64 [n, 2] on the device.
    Asynchronous on the current stream of the device pool."""
    for t, n in ((src_k, "src_k"), (src_v, "src_v"), (dst_k, "dst_k"), (dst_v, "dst_v")):
        _reachable(t, n)
    _dev(src_dst_pairs, "src_dst_pairs")
    dt = src_k.dtype
    if dt not in _CACHE_CODE or any(t.dtype != dt for t in (src_v, dst_k, dst_v)):
        raise ValueError("pools must share one supported dtype")
    if src_k.dim() != 4 or src_v.shape != src_k.shape or dst_k.dim() != 4 or \
            dst_v.shape != dst_k.shape or dst_k.shape[1:] != src_k.shape[1:]:
        raise ValueError("pools must be [num_blocks, num_kv_heads, block_size, head_dim] alike")
    if src_dst_pairs.dtype != torch.int64 or src_dst_pairs.dim() != 2 or \
            src_dst_pairs.shape[1] != 2:
        raise ValueError("src_dst_pairs must be int64 [num_pairs, 2]")
    nsrc, hkv, bs, hd = src_k.shape
    ndst = dst_k.shape[0]
    dev = src_dst_pairs.device
    with torch.cuda.device(dev):
        st = lib.pkv_swap_blocks(_ptr(dst_k), _ptr(dst_v), _ptr(src_k), _ptr(src_v),
                                 _ptr(src_dst_pairs), src_dst_pairs.shape[0], hkv, hd, bs, nsrc,
                                 ndst, _CACHE_CODE[dt], _stream(src_dst_pairs, stream))
    _check("swap_blocks", st)


def reshape_and_cache_fp8(k, v, k_cache, v_cache, slot_mapping, k_scale, v_scale, stream=None):
    """Quantising cache write (``pkv_reshape_and_cache_fp8``): rows of ``k``
    and ``v`` ([num_tokens, Hkv, hd], float32/float16/bfloat16) become E4M3
    codes of ``x / k_scale`` and ``x / v_scale`` in the uint8 caches."""
    for t, n in ((k, "k"), (v, "v"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                 (slot_mapping, "slot_mapping")):
        _dev(t, n)
    if k.dtype not in _DTYPE_CODE or v.dtype != k.dtype:
        raise ValueError("k and v must share one supported dtype")
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise ValueError("8-bit caches must be uint8 tensors of E4M3 codes")
    if k.dim() != 3 or v.shape != k.shape:
        raise ValueError("k and v must both be [num_tokens, num_kv_heads, head_dim]")
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("caches must both be [num_blocks, num_kv_heads, block_size, head_dim]")
    nb, hkv, bs, hd = k_cache.shape
    if k.shape[1:] != (hkv, hd):
        raise ValueError("k/v rows do not match the cache's [num_kv_heads, head_dim]")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (k.shape[0],):
        raise ValueError("slot_mapping must be int64 [num_tokens]")
    with torch.cuda.device(k.device):
        st = lib.pkv_reshape_and_cache_fp8(_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache),
                                           _ptr(slot_mapping), k.shape[0], hkv, hd, bs, nb,
                                           _DTYPE_CODE[k.dtype], ctypes.c_float(k_scale),
                                           ctypes.c_float(v_scale), _stream(k, stream))
    _check("reshape_and_cache_fp8", st)


def paged_attention_decode_fp8(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                               k_scale, v_scale, max_context_len, workspace=None,
                               partition_tokens=0, path=PATH_AUTO, grid=GRID_AUTO, stream=None,
                               kernel_events=None):
    """Decode attention over E4M3 caches (``pkv_paged_attention_decode_fp8``):
    keys and values are ``value(code) * k_scale`` and ``value(code) *
    v_scale``; otherwise as :func:`paged_attention_decode`."""
    for t, n in ((out, "out"), (q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                 (context_lens, "context_lens"), (block_tables, "block_tables")):
        _dev(t, n)
    if q.dtype not in _DTYPE_CODE or out.dtype != q.dtype:
        raise ValueError("q and out must share one supported dtype")
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise ValueError("8-bit caches must be uint8 tensors of E4M3 codes")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2:
        raise ValueError("block_tables must be int32 [num_seqs, max_blocks]")
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must both be [num_seqs, num_q_heads, head_dim]")
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("caches must both be [num_blocks, num_kv_heads, block_size, head_dim]")
    num_seqs, hq, hd = q.shape
    nb, hkv, bs, hd2 = k_cache.shape
    if hd2 != hd:
        raise ValueError("head_dim of q and caches differ")
    if context_lens.dtype != torch.int32 or context_lens.shape != (num_seqs,):
        raise ValueError("context_lens must be int32 [num_seqs]")
    if block_tables.shape[0] != num_seqs:
        raise ValueError("block_tables must have num_seqs rows")
    max_blocks = block_tables.shape[1]
    need = workspace_bytes(num_seqs, hq, hkv, hd, bs, max_blocks, int(max_context_len),
                           _DTYPE_CODE[q.dtype] | KV_E4M3, partition_tokens, path, grid)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with torch.cuda.device(q.device):
        ev0, ev1 = (kernel_events[0].handle, kernel_events[1].handle) if kernel_events \
            else (None, None)
        st = lib.pkv_paged_attention_decode_fp8(
            _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            _ptr(context_lens), ctypes.c_float(scale), ctypes.c_float(k_scale),
            ctypes.c_float(v_scale), num_seqs, hq, hkv, hd, bs, nb, max_blocks,
            int(max_context_len), _DTYPE_CODE[q.dtype], ws_ptr, ws_len, int(partition_tokens),
            int(path), int(grid), ev0, ev1, _stream(q, stream))
    _check("paged_attention_decode_fp8", st)
    return out


def paged_attention_prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start,
                            scale, max_q_len, max_context_len, stream=None, kernel_events=None,
                            k_scale=None, v_scale=None):
    """Causal attention of the last ``n_s`` positions of every sequence over
    its paged KV (``pkv_paged_attention_prefill``).  ``q`` / ``out`` are
    ``[total_q, Hq, hd]``; sequence s owns rows ``query_start[s] ..
    query_start[s+1]`` (int32 [B+1] on the device); ``max_q_len`` is a
    host-side bound of the ``n_s``.  With uint8 caches of E4M3 codes, pass
    ``k_scale`` and ``v_scale`` (``pkv_paged_attention_prefill_fp8``)."""
    for t, n in ((out, "out"), (q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                 (block_tables, "block_tables"), (context_lens, "context_lens"),
                 (query_start, "query_start")):
        _dev(t, n)
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("prefill runs on float16 or bfloat16")
    fp8 = k_scale is not None or v_scale is not None
    if fp8 and (k_scale is None or v_scale is None):
        raise ValueError("8-bit caches need both k_scale and v_scale")
    cache_dtype = torch.uint8 if fp8 else q.dtype
    if out.dtype != q.dtype:
        raise ValueError(f"out dtype {out.dtype} != q dtype {q.dtype}")
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        if t.dtype != cache_dtype:
            raise ValueError(f"{n} dtype {t.dtype}, expected {cache_dtype}")
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must both be [total_q, num_q_heads, head_dim]")
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("caches must both be [num_blocks, num_kv_heads, block_size, head_dim]")
    total_q, hq, hd = q.shape
    nb, hkv, bs, hd2 = k_cache.shape
    if hd2 != hd:
        raise ValueError("head_dim of q and caches differ")
    num_seqs = context_lens.shape[0]
    if context_lens.dtype != torch.int32 or context_lens.dim() != 1:
        raise ValueError("context_lens must be int32 [num_seqs]")
    if query_start.dtype != torch.int32 or query_start.shape != (num_seqs + 1,):
        raise ValueError("query_start must be int32 [num_seqs + 1]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or \
            block_tables.shape[0] != num_seqs:
        raise ValueError("block_tables must be int32 [num_seqs, max_blocks]")
    with torch.cuda.device(q.device):
        ev0, ev1 = (kernel_events[0].handle, kernel_events[1].handle) if kernel_events \
            else (None, None)
        common = (int(max_q_len), hq, hkv, hd, bs, nb, block_tables.shape[1],
                  int(max_context_len), _DTYPE_CODE[q.dtype], ev0, ev1, _stream(q, stream))
        head = (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                _ptr(context_lens), _ptr(query_start), ctypes.c_float(scale))
        if fp8:
            st = lib.pkv_paged_attention_prefill_fp8(*head, ctypes.c_float(k_scale),
                                                     ctypes.c_float(v_scale), num_seqs, total_q,
                                                     *common)
        else:
            st = lib.pkv_paged_attention_prefill(*head, num_seqs, total_q, *common)
    _check("paged_attention_prefill", st)
    return out


def group_tiles(block_tables, context_lens, group_members, block_size, max_context_len,
                tiles=None, tile_start=None, tile_end=None, stream=None):
    """The grouped decode's tile lists built on the device from the block
    tables (``pkv_group_tiles``): returns ``(tiles, tile_start, tile_end)``,
    int32 ``[capacity, 4]``, ``[G]`` and ``[G]`` (group j's rows are
    ``tiles[tile_start[j]:tile_end[j]]``; pass all three to
    :func:`paged_attention_decode_grouped`).  Buffers may be given for reuse."""
    for t, n in ((block_tables, "block_tables"), (context_lens, "context_lens"),
                 (group_members, "group_members")):
        _dev(t, n)
        if t.dtype != torch.int32:
            raise ValueError(f"{n} must be int32")
    if block_tables.dim() != 2 or group_members.dim() != 2:
        raise ValueError("block_tables and group_members must be 2-D")
    num_seqs, max_blocks = block_tables.shape
    if context_lens.shape != (num_seqs,):
        raise ValueError("context_lens must be [num_seqs]")
    num_groups, max_members = group_members.shape
    need = lib.pkv_group_tiles_capacity(num_groups, max_members, int(block_size), max_blocks,
                                        int(max_context_len))
    if need == ctypes.c_size_t(-1).value:
        raise ValueError("invalid sizes for group_tiles")
    dev = block_tables.device
    if tiles is None:
        tiles = torch.empty((max(need, 1), 4), dtype=torch.int32, device=dev)
    if tile_start is None:
        tile_start = torch.empty(max(num_groups, 1), dtype=torch.int32, device=dev)
    if tile_end is None:
        tile_end = torch.empty(max(num_groups, 1), dtype=torch.int32, device=dev)
    if tiles.dtype != torch.int32 or tiles.dim() != 2 or tiles.shape[1] != 4:
        raise ValueError("tiles must be int32 [capacity, 4]")
    for t, n in ((tile_start, "tile_start"), (tile_end, "tile_end")):
        if t.dtype != torch.int32 or t.dim() != 1 or t.shape[0] < num_groups:
            raise ValueError(f"{n} must be int32 [num_groups]")
        _dev(t, n)
    _dev(tiles, "tiles")
    with torch.cuda.device(dev):
        st = lib.pkv_group_tiles(_ptr(block_tables), _ptr(context_lens), _ptr(group_members),
                                 num_seqs, max_blocks, num_groups, max_members, int(block_size),
                                 int(max_context_len), _ptr(tiles), tiles.shape[0],
                                 _ptr(tile_start), _ptr(tile_end), _stream(block_tables, stream))
    _check("group_tiles", st)
    return tiles, tile_start, tile_end


def grouped_workspace_bytes(num_groups, num_kv_heads, head_dim, part_tiles, max_group_tiles):
    n = lib.pkv_paged_attention_grouped_workspace_bytes(num_groups, num_kv_heads, head_dim,
                                                        part_tiles, max_group_tiles)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid arguments for the grouped workspace size")
    return n


def paged_attention_decode_grouped(out, q, k_cache, v_cache, context_lens, group_members,
                                   group_tiles, group_tile_start, scale, max_context_len,
                                   part_tiles=0, max_group_tiles=0, workspace=None,
                                   stream=None, kernel_events=None, k_scale=None, v_scale=None,
                                   group_tile_end=None):
    """Decode attention of sequences that share KV blocks, each shared tile
    read once for its whole group (``pkv_paged_attention_decode_grouped``).
    The rows of every grouped sequence equal :func:`paged_attention_decode`'s.
    ``group_members`` int32 ``[G, M]`` (-1 = empty), ``group_tiles`` int32
    ``[T, 4]`` (block, tile index, member mask, 0), ``group_tile_start`` int32
    ``[G + 1]``, all on the device; build them with
    :func:`paged_kv_cache_389_amd.block_manager.group_tiles` (a prefix
    ``group_tile_start``), or on the device with :func:`group_tiles` (pass its
    ``tile_start`` and ``tile_end`` as ``group_tile_start`` /
    ``group_tile_end``).  With
    ``part_tiles > 0`` each group's list is cut into parts of that many rows
    (``max_group_tiles``: host bound of the groups' row counts) whose states a
    second kernel merges; ``workspace`` (uint8, device) is allocated when None.
    With uint8 caches of E4M3 codes, pass ``k_scale`` and ``v_scale``
    (``pkv_paged_attention_decode_grouped_fp8``)."""
    for t, n in ((out, "out"), (q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                 (context_lens, "context_lens"), (group_members, "group_members"),
                 (group_tiles, "group_tiles"), (group_tile_start, "group_tile_start")):
        _dev(t, n)
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("grouped decode runs on float16 or bfloat16")
    fp8 = k_scale is not None or v_scale is not None
    if fp8 and (k_scale is None or v_scale is None):
        raise ValueError("8-bit caches need both k_scale and v_scale")
    if out.dtype != q.dtype:
        raise ValueError(f"out dtype {out.dtype} != q dtype {q.dtype}")
    cache_dtype = torch.uint8 if fp8 else q.dtype
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        if t.dtype != cache_dtype:
            raise ValueError(f"{n} dtype {t.dtype}, expected {cache_dtype}")
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must both be [num_seqs, num_q_heads, head_dim]")
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("caches must both be [num_blocks, num_kv_heads, block_size, head_dim]")
    num_seqs, hq, hd = q.shape
    nb, hkv, bs, hd2 = k_cache.shape
    if hd2 != hd:
        raise ValueError("head_dim of q and caches differ")
    if context_lens.dtype != torch.int32 or context_lens.shape != (num_seqs,):
        raise ValueError("context_lens must be int32 [num_seqs]")
    for t, n in ((group_members, "group_members"), (group_tiles, "group_tiles"),
                 (group_tile_start, "group_tile_start")):
        if t.dtype != torch.int32:
            raise ValueError(f"{n} must be int32")
    if group_members.dim() != 2:
        raise ValueError("group_members must be [num_groups, max_members]")
    num_groups, max_members = group_members.shape
    if group_tile_end is None and group_tile_start.shape != (num_groups + 1,):
        raise ValueError("group_tile_start must be [num_groups + 1]")
    if group_tile_end is not None:
        _dev(group_tile_end, "group_tile_end")
        if group_tile_end.dtype != torch.int32 or group_tile_start.shape[0] < num_groups or \
                group_tile_end.shape[0] < num_groups:
            raise ValueError("group_tile_start / group_tile_end must be int32 [num_groups]")
    if group_tiles.dim() != 2 or group_tiles.shape[1] != 4:
        raise ValueError("group_tiles must be [total, 4]")
    need = grouped_workspace_bytes(num_groups, hkv, hd, int(part_tiles), int(max_group_tiles))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with torch.cuda.device(q.device):
        ev0, ev1 = (kernel_events[0].handle, kernel_events[1].handle) if kernel_events \
            else (None, None)
        head = (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(context_lens),
                _ptr(group_members), _ptr(group_tiles), _ptr(group_tile_start),
                _ptr(group_tile_end) if group_tile_end is not None else None,
                int(group_tiles.shape[0]), ctypes.c_float(scale))
        tail = (num_seqs, num_groups, max_members, hq, hkv, hd, bs, nb, int(max_context_len),
                _DTYPE_CODE[q.dtype], int(part_tiles), int(max_group_tiles), ws_ptr, ws_len,
                ev0, ev1, _stream(q, stream))
        if fp8:
            st = lib.pkv_paged_attention_decode_grouped_fp8(*head, ctypes.c_float(k_scale),
                                                            ctypes.c_float(v_scale), *tail)
        else:
            st = lib.pkv_paged_attention_decode_grouped(*head, *tail)
    _check("paged_attention_decode_grouped", st)
    return out


def ceiling_stream_read(src, workgroups, sink, stream=None):
    """Read every byte of the contiguous device tensor ``src`` once
    (``pkv_ceiling_stream_read``, a reference read for the practical
    bandwidth ceiling); ``sink`` is a one-element int32 device tensor the
    kernel XORs into."""
    _dev(src, "src")
    _dev(sink, "sink")
    nbytes = src.numel() * src.element_size()
    with torch.cuda.device(src.device):
        st = lib.pkv_ceiling_stream_read(_ptr(src), nbytes, int(workgroups), _ptr(sink),
                                         _stream(src, stream))
    _check("ceiling_stream_read", st)


def ceiling_gather_read(pool, chunks, chunk_bytes, workgroups, sink, pool2=None, cached=False,
                        stream=None):
    """Read the ``chunk_bytes`` chunks of the device tensor ``pool`` (and of
    ``pool2``, same size, when given) that the int32 device tensor ``chunks``
    names (``pkv_ceiling_gather_read``, a reference read for the practical
    ceiling of a paged gather); streaming loads unless ``cached``."""
    _dev(pool, "pool")
    _dev(chunks, "chunks")
    _dev(sink, "sink")
    if chunks.dtype != torch.int32 or chunks.dim() != 1:
        raise ValueError("chunks must be int32 [n]")
    nbytes = pool.numel() * pool.element_size()
    if pool2 is not None:
        _dev(pool2, "pool2")
        if pool2.numel() * pool2.element_size() != nbytes:
            raise ValueError("pool2 must have the size of pool")
    with torch.cuda.device(pool.device):
        st = lib.pkv_ceiling_gather_read(_ptr(pool), _ptr(pool2) if pool2 is not None else None,
                                         nbytes, _ptr(chunks), chunks.numel(), int(chunk_bytes),
                                         1 if cached else 0, int(workgroups), _ptr(sink),
                                         _stream(pool, stream))
    _check("ceiling_gather_read", st)


class HipEvent:
    """A timing hipEvent_t of the HIP runtime that torch loaded, for
    ``kernel_events`` (the library records it; read it with
    :meth:`elapsed_ms`)."""

    _hip = None

    def __init__(self):
        if HipEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            HipEvent._hip = hip
        self.handle = ctypes.c_void_p()
        if HipEvent._hip.hipEventCreate(ctypes.byref(self.handle)) != 0:
            raise PagedKVError("hipEventCreate failed")

    def elapsed_ms(self, end: "HipEvent") -> float:
        """Milliseconds from this event to ``end`` (both recorded; waits for end)."""
        hip = HipEvent._hip
        if hip.hipEventSynchronize(end.handle) != 0:
            raise PagedKVError("hipEventSynchronize failed")
        ms = ctypes.c_float()
        if hip.hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle) != 0:
            raise PagedKVError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        if HipEvent._hip is not None and self.handle:
            HipEvent._hip.hipEventDestroy(self.handle)
