"""Plant mistakes into copies of the decode oracle (on the CPU) and check
that the pins catch each one.  This shows the pins constrain the oracle:
a dropped term, a wrong index or sign, or a transposed operand fails."""

import math

import numpy as np
import pytest

import pins


def _make(kv_of=lambda h, hq, hkv: h // (hq // hkv), scale_fn=lambda s: s,
          block_of=lambda t, bs: t // bs, offset_of=lambda t, bs: t % bs,
          n_tokens=lambda L, bs: L, subtract_max=True, normalise=True,
          values_from_keys=False, sign=1.0, transpose_heads=False):
    """A per-token decode oracle with pluggable pieces (the correct
    arguments reproduce the oracle's definition)."""

    def decode(q, kc, vc, tables, lens, scale, hkv):
        b, hq, hd = q.shape
        out = np.zeros((b, hq, hd))
        for s in range(b):
            for h in range(hq):
                g = kv_of(h, hq, hkv)
                L = n_tokens(int(lens[s]), kc.shape[2])
                if int(lens[s]) == 0:
                    continue
                sc, vals = [], []
                for t in range(L):
                    blk = int(tables[s][block_of(t, kc.shape[2])])
                    off = offset_of(t, kc.shape[2])
                    if transpose_heads:
                        k = np.asarray(kc[blk, off % kc.shape[1], g % kc.shape[2]], float)
                        v = np.asarray(vc[blk, off % kc.shape[1], g % kc.shape[2]], float)
                    else:
                        k = np.asarray(kc[blk, g, off], float)
                        v = np.asarray(vc[blk, g, off], float)
                    sc.append(scale_fn(scale) * float(np.dot(q[s, h], k)))
                    vals.append(k if values_from_keys else v)
                sc = np.array(sc) * sign
                m = sc.max() if subtract_max else 0.0
                w = np.exp(sc - m)
                den = w.sum() if normalise else len(w)
                out[s, h] = (w @ np.array(vals)) / den
        return out

    return decode


MUTANTS = {
    "correct": _make(),
    "group_mapping_modulo": _make(kv_of=lambda h, hq, hkv: h % hkv),
    "scale_dropped": _make(scale_fn=lambda s: 1.0),
    "scale_squared": _make(scale_fn=lambda s: s * s),
    "scale_sqrt": _make(scale_fn=lambda s: math.sqrt(abs(s))),
    "block_offset_swapped": _make(block_of=lambda t, bs: t % bs, offset_of=lambda t, bs: t // bs),
    "offset_off_by_one": _make(offset_of=lambda t, bs: (t + 1) % bs),
    "tail_not_masked": _make(n_tokens=lambda L, bs: -(-L // bs) * bs),
    "tail_dropped": _make(n_tokens=lambda L, bs: max(1, (L // bs) * bs)),
    "last_token_dropped": _make(n_tokens=lambda L, bs: max(1, L - 1)),
    "no_max_subtraction": _make(subtract_max=False),
    "normalised_by_count": _make(normalise=False),
    "values_read_from_keys": _make(values_from_keys=True),
    "score_sign_flipped": _make(sign=-1.0),
    "head_and_slot_axes_transposed": _make(transpose_heads=True),
}


def _caught(decode):
    failures = []
    for pin in pins.ALL_DECODE_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(decode)
        except (AssertionError, IndexError, ValueError, FloatingPointError) as e:
            failures.append((pin.__name__, type(e).__name__))
    return failures


def test_correct_per_token_variant_passes_every_pin():
    assert _caught(MUTANTS["correct"]) == []


@pytest.mark.parametrize("name", [n for n in MUTANTS if n != "correct"])
def test_mutant_is_caught(name):
    assert _caught(MUTANTS[name]), f"no pin caught the planted mistake {name!r}"
