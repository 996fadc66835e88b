"""Oracle: an 8-bit floating-point KV cache (OCP E4M3), in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages give: the broader-context section of "Memory Optimization in
LLM Serving with PagedAttention" names INT8/FP8 quantization of the cache as
a feature of other serving libraries, and nothing more.  Everything below is
therefore a reading, the plainest one that fits the rest of the path:

* Format: the OCP 8-bit E4M3 encoding (the FP8 format gfx950 converts to and
  from natively).  A code is sign (bit 7), a 4-bit exponent field e (bits
  6..3, bias 7) and a 3-bit fraction f (bits 2..0).  e > 0 encodes
  ``(1 + f/8) * 2**(e - 7)``; e == 0 encodes the subnormal ``f/8 * 2**-6``.
  There is no infinity; e == 15 with f == 7 is NaN, so the largest finite
  magnitude is ``1.75 * 2**8 = 448`` (code 0x7E).
* Scaling: one float32 scale for the whole K cache and one for the whole V
  cache.  A stored code represents ``value(code) * scale``.
* Quantisation (what reshape_and_cache writes): the source element is
  widened to float32 and divided by the scale in float32 (round to nearest
  even), and that float32 quotient is encoded: NaN gives 0x7F; a magnitude
  above 448 (infinity included) saturates to 448 with its sign; anything
  else goes to the nearest representable value, ties to the code with an
  even fraction (round to nearest even).  Zero keeps its sign.  The float32
  steps are the precision the device kernel decides the code in, so both
  sides take the same decision.
* Attention over such a cache (decode or prefill) is the plain attention of
  ``decode`` / ``prefill`` over the dequantised values ``value(code) * scale``
  (exact in float64).
"""

import numpy as np

from .cache_ops import reshape_and_cache as _write_rows
from .paged_attention import decode as _decode
from .prefill import prefill as _prefill

NAN_CODE = 0x7F
MAX_CODE = 0x7E      # +448


def e4m3_value(code):
    """float64 value(s) of E4M3 code(s), from the bit fields (NaN for the
    two NaN codes)."""
    c = np.asarray(code, dtype=np.int64) & 0xFF
    sign = np.where(c >> 7 == 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    f = c & 0x7
    normal = (1.0 + f / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (f / 8.0) * 2.0 ** -6
    mag = np.where(e == 0, sub, normal)
    mag = np.where((e == 15) & (f == 7), np.nan, mag)
    return sign * mag


# the 127 finite non-negative magnitudes, code 0x00 .. 0x7E in increasing order
_MAGNITUDES = e4m3_value(np.arange(0, MAX_CODE + 1))


def e4m3_encode(x):
    """E4M3 code(s) of float value(s): NaN -> 0x7F, saturate at 448, else the
    nearest finite value with ties to the even code.  Zero keeps its sign."""
    xs = np.asarray(x, dtype=np.float64)
    flat = xs.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for i0 in range(0, flat.size, 1 << 16):
        x_ = flat[i0:i0 + (1 << 16)]
        nan = np.isnan(x_)
        neg = np.signbit(x_)
        mag = np.minimum(np.abs(np.where(nan, 0.0, x_)), 448.0)
        # distance to every finite magnitude; the nearest wins, and of two
        # equally near codes the even one (adjacent codes differ in parity)
        d = np.abs(mag[:, None] - _MAGNITUDES[None, :])
        best = d.min(axis=1, keepdims=True)
        cand = d == best
        even = cand & (np.arange(MAX_CODE + 1)[None, :] % 2 == 0)
        code = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
        code = code | (neg.astype(np.int64) << 7)
        out[i0:i0 + x_.size] = np.where(nan, NAN_CODE, code).astype(np.uint8)
    return out.reshape(xs.shape)


def quantize(x, scale):
    """Codes of the source values ``x`` (any float dtype, numpy or CPU torch)
    under ``scale``: float32 quotient ``float32(x) / float32(scale)``, then
    ``e4m3_encode``."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float32).numpy()
    except ImportError:  # pragma: no cover
        pass
    x32 = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        q = x32 / np.float32(scale)
    return e4m3_encode(q.astype(np.float64))


def dequantize(codes, scale):
    """float64 values ``value(code) * scale``."""
    return e4m3_value(codes) * float(np.float32(scale))


def reshape_and_cache_fp8(k, v, k_cache, v_cache, slot_mapping, k_scale, v_scale):
    """The quantising cache write: each new token's K and V rows are
    quantised (``quantize``) and their codes written into the token's slot,
    exactly as ``reshape_and_cache`` writes unquantised rows.  ``k_cache`` and
    ``v_cache`` are uint8 arrays ``[num_blocks, num_kv_heads, block_size,
    head_dim]`` updated in place."""
    _write_rows(quantize(k, k_scale), quantize(v, v_scale), k_cache, v_cache, slot_mapping)


def decode_fp8(q, k_codes, v_codes, block_tables, context_lens, scale, k_scale, v_scale,
               num_kv_heads, seqs=None, heads=None):
    """Paged decode attention over E4M3 caches: ``decode`` on the dequantised
    K and V (float64)."""
    return _decode(q, dequantize(k_codes, k_scale), dequantize(v_codes, v_scale), block_tables,
                   context_lens, scale, num_kv_heads, seqs=seqs, heads=heads)


def prefill_fp8(q, k_codes, v_codes, block_tables, context_lens, query_start, scale, k_scale,
                v_scale, num_kv_heads, rows=None, heads=None):
    """Causal paged prefill over E4M3 caches: ``prefill`` on the dequantised K
    and V (float64)."""
    return _prefill(q, dequantize(k_codes, k_scale), dequantize(v_codes, v_scale), block_tables,
                    context_lens, query_start, scale, num_kv_heads, rows=rows, heads=heads)
