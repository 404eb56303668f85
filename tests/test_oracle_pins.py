"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each check is written so that a plausible slip in the oracle (dropped term,
wrong sign, wrong index or pairing, off-by-one position, truncation instead of
round-to-nearest-even) fails at least one of them; test_oracle_mutants.py
plants such slips and confirms it.  No check retypes the oracle's formula:
they use hand-worked fixtures (tests/golden), closed forms, library routines
(torch's float32->bfloat16 conversion, cmath, torch attention), brute force,
and invariants the pages rely on (InferScale review: Theorem 3, Theorem 6 and
the RoPE axiom R_a^T R_b = R_{b-a}).
"""

import cmath
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention, bf16, inject, paged, retrieve, rope

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# bfloat16 rounding
# --------------------------------------------------------------------------

def load_bf16_golden():
    cases = []
    with open(os.path.join(GOLDEN, "bf16_rounding.txt")) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if not line:
                continue
            # value expression, hex bits, then the comment words
            parts = line.split()
            hex_idx = next(i for i, p in enumerate(parts) if p.startswith("0x"))
            expr = " ".join(parts[:hex_idx])
            cases.append((eval(expr, {"__builtins__": {}}, {"float": float}),
                          int(parts[hex_idx], 16)))
    return cases


def check_bf16_golden():
    for value, want in load_bf16_golden():
        got = int(bf16.f64_to_bf16_bits(np.float64(value)))
        assert got == want, (value, hex(got), hex(want))


def check_bf16_exhaustive_roundtrip():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16.bf16_bits_to_f64(bits)
    finite = np.isfinite(vals)
    back = bf16.f64_to_bf16_bits(vals[finite])
    assert np.array_equal(back, bits[finite])
    # value side: the decoded value equals the float32 whose top half is the pattern
    with np.errstate(invalid="ignore"):
        as32 = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(vals[finite], as32[finite])


def check_bf16_midpoints():
    # every pair of adjacent positive finite bf16 values (a, b): the exact
    # midpoint goes to the even pattern; a float64 ulp either side goes to the nearer.
    lo_bits = np.arange(0, 0x7F7F, dtype=np.int64)          # a = lo, b = lo + 1
    a = bf16.bf16_bits_to_f64(lo_bits)
    b = bf16.bf16_bits_to_f64(lo_bits + 1)
    mid = (a + b) / 2.0                                    # exact in float64
    even = np.where(lo_bits % 2 == 0, lo_bits, lo_bits + 1)
    assert np.array_equal(bf16.f64_to_bf16_bits(mid).astype(np.int64), even)
    above = np.nextafter(mid, np.inf)
    below = np.nextafter(mid, -np.inf)
    assert np.array_equal(bf16.f64_to_bf16_bits(above).astype(np.int64), lo_bits + 1)
    assert np.array_equal(bf16.f64_to_bf16_bits(below).astype(np.int64), lo_bits)
    # negative side mirrors the positive side
    assert np.array_equal(bf16.f64_to_bf16_bits(-mid).astype(np.int64), even | 0x8000)


def check_bf16_matches_torch():
    # Special case that reduces to a library routine: for float64 values that
    # are exactly float32, one rounding to bf16 equals torch's float32->bfloat16.
    import torch
    rng = np.random.default_rng(1234)
    raw = rng.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32)
    f32 = raw.view(np.float32)
    f32 = f32[np.isfinite(f32)]
    normal = rng.standard_normal(200_000).astype(np.float32)
    f32 = np.concatenate([f32, normal, normal * 1e-3, normal * 1e30])
    want = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy()
    got = bf16.f64_to_bf16_bits(f32.astype(np.float64))
    assert np.array_equal(got.astype(np.uint16), want.astype(np.uint16))


def test_bf16_golden():
    check_bf16_golden()


def test_bf16_exhaustive_roundtrip():
    check_bf16_exhaustive_roundtrip()


def test_bf16_midpoints_tie_to_even():
    check_bf16_midpoints()


def test_bf16_matches_torch_float32_rounding():
    check_bf16_matches_torch()


def test_ulp_distance_definition():
    # adjacent patterns are 1 apart, across zero +0/-0 coincide, and the
    # smallest positive and negative subnormals are 2 apart
    assert bf16.ulp_distance(0x3F80, 0x3F81) == 1
    assert bf16.ulp_distance(0x0000, 0x8000) == 0
    assert bf16.ulp_distance(0x0001, 0x8001) == 2
    assert bf16.ulp_distance(0x7F7F, 0x7F7E) == 1


# --------------------------------------------------------------------------
# RoPE rotation
# --------------------------------------------------------------------------

def load_rope_golden(name="rope_half_split.txt"):
    cases = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if not line:
                continue
            p, x, y = [s.strip() for s in line.split(";")]
            cases.append((int(p), np.array(x.split(), float), np.array(y.split(), float)))
    return cases


def check_rope_golden():
    for p, x, want in load_rope_golden():
        got = rope.rotate(x, p, 100.0)
        assert np.allclose(got, want, rtol=0, atol=1e-15), (p, x, got, want)


def check_rope_golden_interleaved():
    for p, x, want in load_rope_golden("rope_interleaved.txt"):
        got = rope.rotate(x, p, 100.0, style=rope.INTERLEAVED)
        assert np.allclose(got, want, rtol=0, atol=1e-15), (p, x, got, want)


def _roformer_matrix_rotation(x, p, base):
    """RoFormer's block-diagonal R_p: 2x2 rotation blocks on dims (2j, 2j+1)."""
    d = x.shape[-1]
    r = np.zeros((d, d))
    for j in range(d // 2):
        ang = p * math.pow(base, -2.0 * j / d)
        c, s = math.cos(ang), math.sin(ang)
        r[2 * j, 2 * j], r[2 * j, 2 * j + 1] = c, -s
        r[2 * j + 1, 2 * j], r[2 * j + 1, 2 * j + 1] = s, c
    return r @ x


def check_rope_interleaved_matrix_form():
    rng = np.random.default_rng(17)
    for d, base in ((64, 1e4), (128, 5e5), (8, 10.0)):
        for p in (0, 1, 3, 37, 1000, 13311):
            x = rng.standard_normal(d)
            got = rope.rotate(x, p, base, style=rope.INTERLEAVED)
            want = _roformer_matrix_rotation(x, p, base)
            assert np.allclose(got, want, rtol=0, atol=1e-12 * max(1, p) ** 0.5), (d, p)


def check_rope_styles_are_a_permutation():
    # interleaved = half split conjugated by the permutation that moves the
    # even dims to the first half and the odd dims to the second half
    rng = np.random.default_rng(18)
    for d in (4, 64, 128):
        perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
        x = rng.standard_normal((20, d))
        pos = rng.integers(0, 16384, size=20)
        for scaling in (None, rope.LLAMA31):
            a = rope.rotate(x, pos, 5e5, style=rope.INTERLEAVED, scaling=scaling)
            b = np.empty_like(x)
            b[:, perm] = rope.rotate(x[:, perm], pos, 5e5, scaling=scaling)
            assert np.array_equal(a, b), d


def _matrix_rotation(x, p, base):
    """Textbook form: x' = R_p x, R_p block-diagonal in the half-split pairs."""
    d = x.shape[-1]
    half = d // 2
    r = np.zeros((d, d))
    for j in range(half):
        ang = p * math.pow(base, -2.0 * j / d)
        c, s = math.cos(ang), math.sin(ang)
        r[j, j], r[j, j + half] = c, -s
        r[j + half, j], r[j + half, j + half] = s, c
    return r @ x


def check_rope_matrix_form():
    rng = np.random.default_rng(7)
    for d, base in ((64, 1e4), (128, 5e5), (8, 10.0)):
        for p in (0, 1, 3, 37, 1000, 13311):
            x = rng.standard_normal(d)
            got = rope.rotate(x, p, base)
            want = _matrix_rotation(x, p, base)
            assert np.allclose(got, want, rtol=0, atol=1e-12 * max(1, p) ** 0.5), (d, p)


def check_rope_scalar_d2():
    # D = 2 has one pair with theta_0 = 1: rotation is multiplication by e^{ip}
    rng = np.random.default_rng(8)
    for p in (0, 1, 2, 5, 100, 4095):
        x0, x1 = rng.standard_normal(2)
        z = complex(x0, x1) * cmath.exp(1j * p)
        got = rope.rotate(np.array([x0, x1]), p, 12345.0)
        assert abs(got[0] - z.real) < 1e-13 and abs(got[1] - z.imag) < 1e-13


def check_rope_position_zero_identity():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((5, 3, 128))
    assert np.array_equal(rope.rotate(x, 0, 5e5), x)


def check_rope_norm_per_pair():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((200, 128))
    pos = rng.integers(0, 16384, size=200)
    y = rope.rotate(x, pos, 5e5)
    n_in = x[:, :64] ** 2 + x[:, 64:] ** 2
    n_out = y[:, :64] ** 2 + y[:, 64:] ** 2
    assert np.allclose(n_in, n_out, rtol=1e-13, atol=0)


def check_rope_relocation_composes():
    # R(delta) RoPE(p) = RoPE(p + delta): Theorem 6 relocation
    rng = np.random.default_rng(11)
    x = rng.standard_normal((100, 128))
    p = rng.integers(0, 8000, size=100)
    delta = rng.integers(0, 8000, size=100)
    two_step = rope.rotate(rope.rotate(x, p, 5e5), delta, 5e5)
    one_step = rope.rotate(x, p + delta, 5e5)
    # angle rounding: |error| <~ (p + delta) * 2**-52 per pair
    assert np.allclose(two_step, one_step, rtol=0, atol=1e-11)


def check_rope_relative_position():
    # <RoPE(pq) q, RoPE(pk) k> depends only on pq - pk (axiom R_a^T R_b = R_{b-a})
    rng = np.random.default_rng(12)
    for _ in range(50):
        q = rng.standard_normal(128)
        k = rng.standard_normal(128)
        pq, pk, shift = (int(v) for v in rng.integers(0, 6000, size=3))
        a = np.dot(rope.rotate(q, pq, 5e5), rope.rotate(k, pk, 5e5))
        b = np.dot(rope.rotate(q, pq + shift, 5e5), rope.rotate(k, pk + shift, 5e5))
        assert abs(a - b) < 1e-9 * (1 + abs(a))


def test_rope_golden_half_split():
    check_rope_golden()


def test_rope_golden_interleaved():
    check_rope_golden_interleaved()


def test_rope_interleaved_matches_roformer_matrix():
    check_rope_interleaved_matrix_form()


def test_rope_styles_are_a_permutation():
    check_rope_styles_are_a_permutation()


def test_llama3_regions():
    check_llama3_regions()


def test_llama3_continuous_and_monotone():
    check_llama3_continuous_and_monotone()


def test_rope_matches_matrix_form():
    check_rope_matrix_form()


def test_rope_d2_is_complex_exponential():
    check_rope_scalar_d2()


def test_rope_position_zero_is_identity():
    check_rope_position_zero_identity()


def test_rope_preserves_pair_norm():
    check_rope_norm_per_pair()


def test_rope_relocation_composes():
    check_rope_relocation_composes()


def test_rope_scores_depend_on_relative_position():
    check_rope_relative_position()


def test_rope_frequencies_geometric():
    # closed form: theta_0 = 1, consecutive ratio base**(-2/D), last = base**(-(D-2)/D)
    for d, base in ((64, 1e4), (128, 5e5)):
        f = rope.inv_freq(d, base)
        assert f[0] == 1.0
        assert np.allclose(f[1:] / f[:-1], math.exp(-2.0 / d * math.log(base)), rtol=1e-14)
        assert math.isclose(f[-1], math.exp(-(d - 2) / d * math.log(base)), rel_tol=1e-14)


# --------------------------------------------------------------------------
# Llama 3.1 frequency rule
# --------------------------------------------------------------------------

def check_llama3_regions():
    # Closed form of the three regions for D = 128, base 5e5, W = 8192, low 1,
    # high 4: f_j is kept while 2 pi base^(2j/D) < W/4, divided by 8 once
    # 2 pi base^(2j/D) > W/1, blended in between.  The boundaries in j come
    # from logarithms, not from the oracle.
    d, base, sc = 128, 5e5, rope.LLAMA31
    j_keep = (d / 2) * math.log(sc.original_max_position / sc.high_freq_factor / (2 * math.pi)) \
        / math.log(base)
    j_div = (d / 2) * math.log(sc.original_max_position / sc.low_freq_factor / (2 * math.pi)) \
        / math.log(base)
    plain = rope.inv_freq(d, base)
    scaled = rope.inv_freq(d, base, sc)
    n_keep = n_div = n_mid = 0
    for j in range(d // 2):
        if j < j_keep:
            assert scaled[j] == plain[j], j
            n_keep += 1
        elif j > j_div:
            assert scaled[j] == plain[j] / sc.factor, j   # exact: a power-of-two divide
            n_div += 1
        else:
            assert plain[j] / sc.factor < scaled[j] < plain[j], j
            n_mid += 1
    assert (n_keep, n_mid, n_div) == (29, 6, 29)
    # no rule: the plain frequencies; factor 1: nothing changes anywhere
    same = rope.Llama3Scaling(1.0, 1.0, 4.0, 8192)
    assert np.array_equal(rope.inv_freq(d, base, same), plain)


def check_llama3_continuous_and_monotone():
    from decimal import Decimal
    sc = rope.LLAMA31
    # the blend meets the kept value at wavelength W/high and the divided
    # value at W/low (continuity at both ends of the middle region)
    for w_edge, outer in ((sc.original_max_position / sc.high_freq_factor, 1.0),
                          (sc.original_max_position / sc.low_freq_factor, 1.0 / sc.factor)):
        f_edge = 2 * math.pi / w_edge
        for rel in (1 + 1e-9, 1 - 1e-9):
            f = Decimal(repr(f_edge * rel))
            got = float(rope.scaled_frequency(f, sc)) / float(f)
            assert abs(got - outer) < 1e-7, (w_edge, rel, got)
    # f' is increasing in f over a fine grid spanning all three regions
    fs = np.geomspace(2 * math.pi / 20000, 2 * math.pi / 1000, 4000)
    vals = [float(rope.scaled_frequency(Decimal(repr(float(f))), sc)) for f in fs]
    assert all(b > a for a, b in zip(vals, vals[1:]))


# --------------------------------------------------------------------------
# positions and slots
# --------------------------------------------------------------------------

def load_slot_golden():
    bs, facts, reqs, toks = None, {}, [], []
    with open(os.path.join(GOLDEN, "slot_mapping.txt")) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if not line:
                continue
            if line.startswith("fact "):
                _, fid, row, ln = line.split()
                facts[int(fid)] = (int(row), int(ln))
            elif line.startswith("request "):
                pre, ids, bt = line[len("request "):].split(";")
                reqs.append(([int(v) for v in ids.split()], int(pre),
                             [int(v) for v in bt.split()]))
            elif line.startswith("token "):
                toks.append(tuple(int(v) for v in line.split()[1:]))
            else:
                bs = int(line)
    return bs, facts, reqs, toks


def check_slot_golden():
    bs, facts, reqs, toks = load_slot_golden()
    src, pos, slot = paged.token_mapping(reqs, facts, bs)
    assert list(zip(src, pos, slot)) == toks


def _brute_force_mapping(requests, fact_rows, block_size):
    """Independent derivation: lay every request out as a list of logical
    tokens (prefix placeholders, then each fact's rows), and list the
    physical slots of its blocks in logical order; token i sits in slot i."""
    out = []
    for fact_ids, prefix, bt in requests:
        logical = [None] * prefix
        for f in fact_ids:
            r0, ln = fact_rows[f]
            logical.extend(range(r0, r0 + ln))
        phys = [b * block_size + o for b in bt for o in range(block_size)]
        for i, row in enumerate(logical):
            if row is not None:
                out.append((row, i, phys[i]))
    return out


def check_slot_brute_force():
    rng = np.random.default_rng(13)
    for _ in range(200):
        bs = int(rng.choice([1, 2, 3, 4, 16, 32]))
        n_facts = int(rng.integers(1, 12))
        lens = rng.integers(1, 20, size=n_facts)
        order = rng.permutation(n_facts)
        rows, r = {}, 0
        for f in order:
            rows[int(f) + 100] = (r, int(lens[f]))
            r += int(lens[f])
        nblk = 400
        perm = rng.permutation(nblk)
        reqs, cursor = [], 0
        for _ in range(int(rng.integers(1, 4))):
            k = int(rng.integers(1, n_facts + 1))
            ids = [int(v) + 100 for v in rng.choice(n_facts, size=k, replace=True)]
            prefix = int(rng.integers(0, 40))
            total = prefix + sum(rows[i][1] for i in ids)
            need = -(-total // bs) + int(rng.integers(0, 2))
            reqs.append((ids, prefix, [int(b) for b in perm[cursor:cursor + need]]))
            cursor += need
        src, pos, slot = paged.token_mapping(reqs, rows, bs)
        assert list(zip(src, pos, slot)) == _brute_force_mapping(reqs, rows, bs)
        # injective, and never in a prefix slot
        assert len(set(slot)) == len(slot)


def test_slot_golden():
    check_slot_golden()


def test_slot_brute_force():
    check_slot_brute_force()


# --------------------------------------------------------------------------
# inject end to end (tiny), Theorem 6 and Theorem 3
# --------------------------------------------------------------------------

def _tiny_case(seed=0, num_layers=2, H=2, D=64, bs=16, base=1e4):
    rng = np.random.default_rng(seed)
    n_facts = 12
    lens = rng.integers(3, 30, size=n_facts)
    rows, r = {}, 0
    for f in rng.permutation(n_facts):
        rows[int(f)] = (r, int(lens[f]))
        r += int(lens[f])
    cap = r
    k_ar = bf16.f64_to_bf16_bits(rng.standard_normal((num_layers, cap, H, D)))
    v_ar = bf16.f64_to_bf16_bits(rng.standard_normal((num_layers, cap, H, D)))
    ids = [int(v) for v in rng.choice(n_facts, size=5, replace=False)]
    prefix = 32
    total = prefix + sum(rows[i][1] for i in ids) + 4
    bt = [int(b) for b in rng.permutation(64)[: -(-total // bs)]]
    return dict(rows=rows, k=k_ar, v=v_ar, ids=ids, prefix=prefix, bt=bt, bs=bs,
                base=base, L=num_layers, H=H, D=D)


def check_inject_equals_encode_in_place():
    c = _tiny_case()
    img_k = inject.PagedImage(c["L"], c["bt"], c["bs"], c["H"], c["D"], 0x7F7F)
    img_v = inject.PagedImage(c["L"], c["bt"], c["bs"], c["H"], c["D"], 0x7F7F)
    n = inject.inject(c["k"], c["v"], c["rows"], [(c["ids"], c["prefix"], c["bt"])],
                      c["bs"], c["base"], img_k, img_v)
    assert n == sum(c["rows"][i][1] for i in c["ids"])
    # dense in-place sequence, K rotated by the textbook matrix at each absolute position
    p = c["prefix"]
    written = set()
    for f in c["ids"]:
        r0, ln = c["rows"][f]
        for t in range(ln):
            pos = p + t
            blk, off = c["bt"][pos // c["bs"]], pos % c["bs"]
            written.add((blk, off))
            for layer in range(c["L"]):
                x = bf16.bf16_bits_to_f64(c["k"][layer, r0 + t])
                exact = np.stack([_matrix_rotation(x[h], pos, c["base"]) for h in range(c["H"])])
                got_bits = img_k.data[layer, img_k.index[blk], off]
                got = bf16.bf16_bits_to_f64(got_bits)
                # correctly rounded: within half a bf16 ulp of the exact value
                ulp = np.exp2(np.floor(np.log2(np.abs(got))) - 7)
                assert np.all(np.abs(got - exact) <= 0.5 * ulp * (1 + 1e-9))
                assert np.array_equal(img_v.data[layer, img_v.index[blk], off],
                                      c["v"][layer, r0 + t])
        p += ln
    # every other slot of the listed blocks keeps the sentinel
    for i, blk in enumerate(img_k.block_ids):
        for off in range(c["bs"]):
            if (blk, off) not in written:
                assert np.all(img_k.data[:, i, off] == 0x7F7F)
                assert np.all(img_v.data[:, i, off] == 0x7F7F)


def test_inject_equals_encode_in_place():
    check_inject_equals_encode_in_place()


def check_chunk_local_relocation():
    """A store of keys already rotated at chunk-local positions 0 .. len-1:
    injection applies R(s), s = the fact's first serving position.
    (1) a fact injected at position 0 comes out bit for bit as stored;
    (2) every key is the correctly rounded R(s) of its stored value (textbook
        matrix);
    (3) against the pre-RoPE store (Theorem 6: R(s) R(t) = R(s + t)) the
        result differs only by the one extra rounding of the stored key."""
    c = _tiny_case(seed=3)
    L, H, D, bs, base = c["L"], c["H"], c["D"], c["bs"], c["base"]
    for style in (rope.HALF_SPLIT, rope.INTERLEAVED):
        mat = _matrix_rotation if style == rope.HALF_SPLIT else _roformer_matrix_rotation
        # the chunk-local store: each fact's keys rotated to t = 0 .. len-1, rounded once
        k_local = np.empty_like(c["k"])
        for f, (r0, ln) in c["rows"].items():
            t = np.arange(ln)[None, :, None, None]
            k_local[:, r0:r0 + ln] = inject.rotate_k_bits(c["k"][:, r0:r0 + ln], t[..., 0], base,
                                                          style=style)
        for prefix in (0, c["prefix"]):
            req = [(c["ids"], prefix, c["bt"])]
            imgs = {}
            for name, arena, local in (("pre", c["k"], False), ("local", k_local, True)):
                ik = inject.PagedImage(L, c["bt"], bs, H, D, 0x7F7F)
                iv = inject.PagedImage(L, c["bt"], bs, H, D, 0x7F7F)
                inject.inject(arena, c["v"], c["rows"], req, bs, base, ik, iv, style=style,
                              chunk_local=local)
                imgs[name] = ik
            p = prefix
            for i, f in enumerate(c["ids"]):
                r0, ln = c["rows"][f]
                for t in range(ln):
                    s = paged.slot_of(p + t, c["bt"], bs)
                    for layer in range(L):
                        got_bits = imgs["local"].row(layer, s)
                        if p == 0:
                            assert np.array_equal(got_bits, k_local[layer, r0 + t])
                        got = bf16.bf16_bits_to_f64(got_bits)
                        stored = bf16.bf16_bits_to_f64(k_local[layer, r0 + t])
                        exact = np.stack([mat(stored[h], p, base) for h in range(H)])
                        ulp = np.exp2(np.floor(np.log2(np.abs(got))) - 7)
                        assert np.all(np.abs(got - exact) <= 0.5 * ulp * (1 + 1e-9))
                        pre = bf16.bf16_bits_to_f64(imgs["pre"].row(layer, s))
                        x = bf16.bf16_bits_to_f64(c["k"][layer, r0 + t])
                        first, second = rope.pair_indices(D, style)
                        norm = np.hypot(x[:, first], x[:, second])
                        bound = 3 * 2.0 ** -8 * np.concatenate([norm, norm], axis=-1)
                        diff = np.abs(got - pre)
                        order = np.concatenate([first, second])
                        assert np.all(diff[:, order] <= bound), (style, prefix, f, t)
                p += ln
            assert prefix == 0 or p > c["prefix"]


def test_chunk_local_relocation():
    check_chunk_local_relocation()


def check_rotation_positions():
    # pre-RoPE: the serving position; chunk-local: serving position minus the
    # token's index in its fact (so that R(rotation) R(index) = R(position))
    c = _tiny_case(seed=4)
    req = [(c["ids"], c["prefix"], c["bt"]), (c["ids"][::-1], 7, c["bt"])]
    _, pos, _ = paged.token_mapping(req, c["rows"], c["bs"])
    assert paged.rotation_positions(req, c["rows"], False) == pos
    local = paged.rotation_positions(req, c["rows"], True)
    idx = [t for ids, _, _ in req for f in ids for t in range(c["rows"][f][1])]
    assert [a + t for a, t in zip(local, idx)] == pos


def test_rotation_positions():
    check_rotation_positions()


def check_attention_matches_torch():
    import torch
    rng = np.random.default_rng(14)
    tq, tk, hq, hkv, d = 4, 23, 8, 2, 64
    q = rng.standard_normal((tq, hq, d))
    k = rng.standard_normal((tk, hkv, d))
    v = rng.standard_normal((tk, hkv, d))
    k_pos = np.arange(tk)
    q_pos = np.arange(tk - tq, tk)
    got = attention.causal_gqa(q, q_pos, k, v, k_pos)
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(np.repeat(k, hq // hkv, axis=1)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(np.repeat(v, hq // hkv, axis=1)).permute(1, 0, 2)[None]
    mask = torch.from_numpy(k_pos[None, :] <= q_pos[:, None])
    want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    assert np.allclose(got, want[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_attention_matches_torch():
    check_attention_matches_torch()


def check_theorem3_injected_equals_in_place():
    """Brute-force attention over the injected paged cache equals attention
    over the same tokens encoded in place (prefix, facts, query)."""
    c = _tiny_case(seed=3, num_layers=1)
    rng = np.random.default_rng(15)
    H, D, bs, base = c["H"], c["D"], c["bs"], c["base"]
    P, Q, HQ = c["prefix"], 4, 8
    pre_k = bf16.f64_to_bf16_bits(rng.standard_normal((P, H, D)))
    pre_v = bf16.f64_to_bf16_bits(rng.standard_normal((P, H, D)))
    qk = bf16.f64_to_bf16_bits(rng.standard_normal((Q, H, D)))
    qv = bf16.f64_to_bf16_bits(rng.standard_normal((Q, H, D)))
    qq = rng.standard_normal((Q, HQ, D))
    n_fact_tok = sum(c["rows"][i][1] for i in c["ids"])
    q_pos = np.arange(P + n_fact_tok, P + n_fact_tok + Q)

    # in-place encoding of the whole prompt (textbook matrix rotation, one rounding)
    seq_k, seq_v = [], []
    for t in range(P):
        seq_k.append(np.stack([_matrix_rotation(bf16.bf16_bits_to_f64(pre_k[t, h]), t, base)
                               for h in range(H)]))
        seq_v.append(bf16.bf16_bits_to_f64(pre_v[t]))
    pos = P
    for f in c["ids"]:
        r0, ln = c["rows"][f]
        for t in range(ln):
            x = bf16.bf16_bits_to_f64(c["k"][0, r0 + t])
            seq_k.append(np.stack([_matrix_rotation(x[h], pos, base) for h in range(H)]))
            seq_v.append(bf16.bf16_bits_to_f64(c["v"][0, r0 + t]))
            pos += 1
    for t in range(Q):
        seq_k.append(np.stack([_matrix_rotation(bf16.bf16_bits_to_f64(qk[t, h]), q_pos[t], base)
                               for h in range(H)]))
        seq_v.append(bf16.bf16_bits_to_f64(qv[t]))
    seq_k = bf16.bf16_bits_to_f64(bf16.f64_to_bf16_bits(np.array(seq_k)))
    seq_v = np.array(seq_v)
    q_rot = np.stack([np.stack([_matrix_rotation(qq[t, h], q_pos[t], base) for h in range(HQ)])
                      for t in range(Q)])
    out_in_place = attention.causal_gqa(q_rot, q_pos, seq_k, seq_v, np.arange(len(seq_k)))

    # injected: prefix and query slots hold their own (rotated) K/V; facts come from inject
    img_k = inject.PagedImage(1, c["bt"], bs, H, D, 0x7F7F)
    img_v = inject.PagedImage(1, c["bt"], bs, H, D, 0x7F7F)
    for t in range(P):
        img_k.row(0, paged.slot_of(t, c["bt"], bs))[...] = inject.rotate_k_bits(pre_k[t], t, base)
        img_v.row(0, paged.slot_of(t, c["bt"], bs))[...] = pre_v[t]
    for t in range(Q):
        s = paged.slot_of(q_pos[t], c["bt"], bs)
        img_k.row(0, s)[...] = inject.rotate_k_bits(qk[t], q_pos[t], base)
        img_v.row(0, s)[...] = qv[t]
    inject.inject(c["k"], c["v"], c["rows"], [(c["ids"], P, c["bt"])], bs, base, img_k, img_v)
    total = P + n_fact_tok + Q
    k_ctx = np.array([bf16.bf16_bits_to_f64(img_k.row(0, paged.slot_of(t, c["bt"], bs)))
                      for t in range(total)])
    v_ctx = np.array([bf16.bf16_bits_to_f64(img_v.row(0, paged.slot_of(t, c["bt"], bs)))
                      for t in range(total)])
    out_injected = attention.causal_gqa(q_rot, q_pos, k_ctx, v_ctx, np.arange(total))
    assert np.array_equal(k_ctx, seq_k)
    assert np.array_equal(v_ctx, seq_v)
    assert np.allclose(out_injected, out_in_place, rtol=0, atol=1e-14)


def test_theorem3_injected_equals_in_place():
    check_theorem3_injected_equals_in_place()


# --------------------------------------------------------------------------
# retrieval (exact top-k by inner product)
# --------------------------------------------------------------------------

def check_retrieve_scores_exact():
    # bf16 products are exact in float64; math.fsum gives the correctly
    # rounded sum, so the float64 dot product may differ only by its own
    # rounding (<= E * 2^-53 * sum |products|)
    import math as _m
    rng = np.random.default_rng(16)
    for E in (8, 512, 1536):
        q = bf16.f64_to_bf16_bits(rng.standard_normal(E) / np.sqrt(E))
        e = bf16.f64_to_bf16_bits(rng.standard_normal((7, E)) / np.sqrt(E))
        got = retrieve.scores(q, e)
        qf, ef = bf16.bf16_bits_to_f64(q), bf16.bf16_bits_to_f64(e)
        for f in range(7):
            prods = [float(a) * float(b) for a, b in zip(qf, ef[f])]
            exact = _m.fsum(prods)
            bound = E * 2.0 ** -53 * sum(abs(p) for p in prods)
            assert abs(got[f] - exact) <= bound, (E, f, got[f], exact)


def check_retrieve_topk_golden():
    # hand-worked: scores 0.5, 0.9, 0.9, 0.1, 0.9 -> best three are the 0.9s in id order
    s = [0.5, 0.9, 0.9, 0.1, 0.9]
    assert list(retrieve.topk(s, 3)) == [1, 2, 4]
    assert list(retrieve.topk(s, 4)) == [1, 2, 4, 0]
    assert list(retrieve.topk([-1.0, -0.5, -2.0], 2)) == [1, 0]


def check_retrieve_topk_brute_force():
    rng = np.random.default_rng(17)
    for _ in range(100):
        F = int(rng.integers(1, 300))
        k = int(rng.integers(1, F + 1))
        s = np.round(rng.standard_normal(F), int(rng.integers(0, 3)))  # rounding makes ties
        want = sorted(range(F), key=lambda f: (-s[f], f))[:k]
        got = list(retrieve.topk(s, k))
        assert got == want
        if k < F:
            rest = np.setdiff1d(np.arange(F), got)
            assert s[got].min() >= s[rest].max()


def check_retrieve_topk_nan_last():
    # hand-derived: a NaN score ranks below every number; NaNs by index
    nan = float("nan")
    assert list(retrieve.topk([nan, 0.5, nan, 0.7, -1.0], 5)) == [3, 1, 4, 0, 2]
    assert list(retrieve.topk([nan, nan, -3.0], 2)) == [2, 0]


def test_retrieve_scores_exact():
    check_retrieve_scores_exact()


def test_retrieve_topk_nan_last():
    check_retrieve_topk_nan_last()


def test_retrieve_topk_golden():
    check_retrieve_topk_golden()


def test_retrieve_topk_brute_force():
    check_retrieve_topk_brute_force()


ALL_CHECKS = [
    check_rope_golden_interleaved, check_rope_interleaved_matrix_form,
    check_rope_styles_are_a_permutation, check_llama3_regions,
    check_llama3_continuous_and_monotone, check_chunk_local_relocation,
    check_rotation_positions,
    check_retrieve_scores_exact, check_retrieve_topk_golden, check_retrieve_topk_brute_force,
    check_retrieve_topk_nan_last,
    check_bf16_golden, check_bf16_exhaustive_roundtrip, check_bf16_midpoints,
    check_bf16_matches_torch, check_rope_golden, check_rope_matrix_form,
    check_rope_scalar_d2, check_rope_position_zero_identity, check_rope_norm_per_pair,
    check_rope_relocation_composes, check_rope_relative_position, check_slot_golden,
    check_slot_brute_force, check_inject_equals_encode_in_place,
    check_attention_matches_torch, check_theorem3_injected_equals_in_place,
]
