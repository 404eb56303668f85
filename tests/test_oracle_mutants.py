"""Planted mistakes in the oracle (on the CPU) must be caught by the pins.

Each mutant replaces one oracle function with a plausible slip; the test
asserts that at least one pin in test_oracle_pins fails under it.  This shows
the pins constrain the oracle rather than restate it.
"""

import numpy as np
import pytest

from oracle import bf16, paged, retrieve, rope

import test_oracle_pins as pins


def _rotate_sign_flipped(x, pos, base, style=rope.HALF_SPLIT, scaling=None):
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    w = np.conj(rope.rotation_factors(pos, x.shape[-1], base))
    z = x[..., :half] + 1j * x[..., half:]
    zr = z * w
    return np.concatenate([zr.real, zr.imag], axis=-1)


def _rotate_interleaved(x, pos, base, style=rope.HALF_SPLIT, scaling=None):
    # GPT-J pairing (2j, 2j+1) instead of the half split
    x = np.asarray(x, dtype=np.float64)
    w = rope.rotation_factors(pos, x.shape[-1], base)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    zr = z * w
    out = np.empty_like(x)
    out[..., 0::2] = zr.real
    out[..., 1::2] = zr.imag
    return out


def _inv_freq_wrong_exponent(head_dim, base, scaling=None):
    j = np.arange(head_dim // 2, dtype=np.float64)
    return np.float64(base) ** (-j / head_dim)


def _rotate_dropped_term(x, pos, base, style=rope.HALF_SPLIT, scaling=None):
    # x'[j] = x[j] cos (the -x[j+D/2] sin term dropped)
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    w = rope.rotation_factors(pos, x.shape[-1], base)
    out = np.empty_like(x)
    out[..., :half] = x[..., :half] * w.real
    out[..., half:] = x[..., half:] * w.real + x[..., :half] * w.imag
    return out


_rotate_orig = rope.rotate


def _rotate_interleaved_swapped(x, pos, base, style=rope.HALF_SPLIT, scaling=None):
    # interleaved pairs taken as x[2j+1] + i x[2j]
    x = np.asarray(x, dtype=np.float64)
    if style != rope.INTERLEAVED:
        return _rotate_orig(x, pos, base, style=style, scaling=scaling)
    y = x.copy()
    y[..., 0::2], y[..., 1::2] = x[..., 1::2], x[..., 0::2]
    r = _rotate_orig(y, pos, base, style=style, scaling=scaling)
    out = r.copy()
    out[..., 0::2], out[..., 1::2] = r[..., 1::2], r[..., 0::2]
    return out


_scaled_orig = rope.scaled_frequency


def _llama3_low_high_swapped(f, sc):
    return _scaled_orig(f, rope.Llama3Scaling(sc.factor, sc.high_freq_factor,
                                              sc.low_freq_factor, sc.original_max_position))


def _llama3_multiplied(f, sc):
    return _scaled_orig(f, rope.Llama3Scaling(1.0 / sc.factor, sc.low_freq_factor,
                                              sc.high_freq_factor, sc.original_max_position))


def _llama3_blend_reversed(f, sc):
    from decimal import Decimal
    w_orig = Decimal(sc.original_max_position)
    lo, hi = Decimal(repr(sc.low_freq_factor)), Decimal(repr(sc.high_freq_factor))
    factor = Decimal(repr(sc.factor))
    wavelen = 2 * Decimal("3.14159265358979323846264338327950288") / f
    if wavelen < w_orig / hi:
        return f
    if wavelen > w_orig / lo:
        return f / factor
    m = (w_orig / wavelen - lo) / (hi - lo)
    return m * f / factor + (1 - m) * f


def _rotation_positions_serving(requests, fact_rows, chunk_local=False):
    # ignores the chunk-local layout: rotates by the serving position
    out = []
    for fact_ids, prefix_len, _ in requests:
        lengths = [fact_rows[int(f)][1] for f in fact_ids]
        for positions in paged.fact_positions(prefix_len, lengths):
            out.extend(positions)
    return out


def _round_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        f = x.astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _round_half_up(x):
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.ldexp(np.floor(np.ldexp(m, 8) + 0.5), e - 8)
    with np.errstate(over="ignore", invalid="ignore"):
        f = np.where(np.isfinite(x), r, x).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _positions_off_by_one(prefix_len, fact_lengths):
    out, p = [], int(prefix_len) + 1
    for length in fact_lengths:
        out.append(list(range(p, p + int(length))))
        p += int(length)
    return out


def _positions_sorted_facts(prefix_len, fact_lengths):
    # facts placed by length instead of in list order
    order = sorted(range(len(fact_lengths)), key=lambda i: fact_lengths[i])
    starts, p = {}, int(prefix_len)
    for i in order:
        starts[i] = p
        p += int(fact_lengths[i])
    return [list(range(starts[i], starts[i] + int(fact_lengths[i])))
            for i in range(len(fact_lengths))]


def _slot_logical(pos, block_table, block_size):
    # forgets the block table (logical == physical)
    return int(pos)


def _slot_swapped(pos, block_table, block_size):
    pos = int(pos)
    return int(block_table[pos % len(block_table)]) * block_size + pos // len(block_table)


def _topk_ties_by_larger_id(score, k):
    score = np.asarray(score, dtype=np.float64)
    idx = np.arange(len(score))
    return np.lexsort((-idx, -score))[:k]


def _topk_ascending(score, k):
    score = np.asarray(score, dtype=np.float64)
    return np.lexsort((np.arange(len(score)), score))[:k]


def _scores_drop_last_dim(q_bits, emb_bits):
    q = bf16.bf16_bits_to_f64(q_bits)
    e = bf16.bf16_bits_to_f64(emb_bits)
    return e[:, :-1] @ q[:-1]


MUTANTS = [
    ("topk ties by larger id", retrieve, "topk", _topk_ties_by_larger_id),
    ("topk ascending", retrieve, "topk", _topk_ascending),
    ("scores drop a term", retrieve, "scores", _scores_drop_last_dim),
    ("rope sign flipped", rope, "rotate", _rotate_sign_flipped),
    ("rope interleaved pairing", rope, "rotate", _rotate_interleaved),
    ("rope frequency exponent", rope, "inv_freq", _inv_freq_wrong_exponent),
    ("rope dropped sin term", rope, "rotate", _rotate_dropped_term),
    ("interleaved pair swapped", rope, "rotate", _rotate_interleaved_swapped),
    ("llama3 low/high swapped", rope, "scaled_frequency", _llama3_low_high_swapped),
    ("llama3 multiplies", rope, "scaled_frequency", _llama3_multiplied),
    ("llama3 blend reversed", rope, "scaled_frequency", _llama3_blend_reversed),
    ("chunk-local rotated by position", paged, "rotation_positions",
     _rotation_positions_serving),
    ("bf16 truncation", bf16, "f64_to_bf16_bits", _round_truncate),
    ("bf16 round half up", bf16, "f64_to_bf16_bits", _round_half_up),
    ("positions off by one", paged, "fact_positions", _positions_off_by_one),
    ("facts reordered", paged, "fact_positions", _positions_sorted_facts),
    ("slot ignores block table", paged, "slot_of", _slot_logical),
    ("slot index swapped", paged, "slot_of", _slot_swapped),
]


@pytest.mark.parametrize("name,module,attr,fn", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(monkeypatch, name, module, attr, fn):
    monkeypatch.setattr(module, attr, fn)
    rope._inv_freq.cache_clear()   # memoised frequencies must see the mutant
    failures = []
    try:
        for check in pins.ALL_CHECKS:
            try:
                with np.errstate(all="ignore"):
                    check()
            except AssertionError:
                failures.append(check.__name__)
            except (IndexError, KeyError, ValueError):
                failures.append(check.__name__ + " (error)")
    finally:
        rope._inv_freq.cache_clear()
    assert failures, f"no pin caught mutant: {name}"
