"""Host checks of the shortcuts the worker-sum kernels take for sub-byte
codes, each claimed to give exactly what decoding every term and adding it
in worker order gives:

* TernGrad: a 2-bit code placed at the top of an fp16 half is the factor
  f in {+0, 2, -0, -2}; the kernel adds fma(f, fl(s/2), acc), which is
  acc + DQ rounded once as long as fl(s/2) is exact, and it takes that form
  only for the scales its guard admits.  Code 2 (never emitted; it decodes
  to +0) reads as -0 there, and the kernel sums again, term by term, only
  the sums that end at -0: checked by brute force over short term
  sequences that every other sum is the rule's sum bit for bit.
* INT2: two adjacent codes become the low address byte 8 (c0 + 4 c1) of a
  16-entry table of decoded pairs; the byte extraction, the v_perm that
  puts it over the table's base, and the lanes' table layout are emulated
  here on every byte value.

The formulas are the kernels' own, evaluated with numpy float32 (IEEE,
correctly rounded) and Python integers."""
import itertools

import numpy as np
import pytest


def f32(bits):
    return np.array(bits, dtype=np.uint32).view(np.float32)


def bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


# ------------------------------------------------------------------ TernGrad


def test_ternary_codes_as_fp16_top_bits():
    want = {0: (0.0, False), 1: (2.0, False), 2: (0.0, True), 3: (-2.0, True)}
    for code, (val, neg) in want.items():
        h = np.array([code << 14], dtype=np.uint16).view(np.float16)[0]
        assert float(h) == val and bool(np.signbit(h)) == neg


def test_ternary_pair_words_hold_codes_j_and_j_plus_8():
    rng = np.random.default_rng(1)
    words = [int(w) for w in rng.integers(0, 2**32, 20000, dtype=np.uint64)] + [0, 0xFFFFFFFF, 0xAAAAAAAA, 0x55555555]
    for w in words:
        for j in range(8):
            y = ((w << (14 - 2 * j)) & 0xFFFFFFFF) & 0xC000C000
            assert y & 0xFFFF == ((w >> (2 * j)) & 3) << 14
            assert y >> 16 == ((w >> (2 * j + 16)) & 3) << 14


def fast_guard(b):
    """The kernel's test for the fma form: not (non-finite, negative or
    below 2^-125 but not zero)."""
    b = np.asarray(b, dtype=np.uint32)
    exact = (b >= 0x7F800000) | ((b - np.uint32(1)) < np.uint32(0x00FFFFFF))
    return ~exact


def test_ternary_half_scale_exact_where_the_guard_admits():
    # every pattern below 2^-124 (the boundary region), and a spread of the rest
    lo = np.arange(0, 0x02000000, dtype=np.uint32)
    rng = np.random.default_rng(2)
    rest = rng.integers(0x02000000, 0x80000000, 4_000_000, dtype=np.uint64).astype(np.uint32)
    edges = np.array([0x7F7FFFFF, 0x7F800000, 0x7FC00000, 0x80000000, 0x80800000, 0xFF7FFFFF], np.uint32)
    b = np.concatenate([lo, rest, edges])
    s = b.view(np.float32)
    ok = fast_guard(b)
    with np.errstate(over="ignore", invalid="ignore"):
        h = s * np.float32(0.5)
        back = h * np.float32(2.0)
    # admitted: s/2 exact (doubling gives s back) and s >= +0
    assert np.all(bits(back[ok]) == b[ok])
    assert not np.any(np.signbit(s[ok]))
    # the guard is needed: some small scales lose their last bit when halved
    small = (b > 0) & (b < 0x01000000)
    assert np.any(bits(back[small]) != b[small])
    assert not np.any(ok[small])


def rule_term(code, s):
    s = np.float32(s)
    if code & 1:
        return -s if code & 2 else s
    return np.float32(0.0)


def raw_term(code, s):
    # the fma form's term f * (s/2), f the fp16 value of the raw code
    f = np.float32(np.array([code << 14], dtype=np.uint16).view(np.float16)[0])
    return f * (np.float32(s) * np.float32(0.5))


def test_ternary_raw_codes_differ_from_the_rule_only_at_negative_zero():
    scales = [0.0, 1.0, 3.0, 0.75]
    starts = [0.0, -0.0, 1.0, -1.0, -3.0, 0.5]
    terms = [(c, s) for c in range(4) for s in scales]
    differ = 0
    for length in range(1, 4):
        for seq in itertools.product(terms, repeat=length):
            for a0 in starts:
                a_rule = np.float32(a0)
                a_raw = np.float32(a0)
                for c, s in seq:
                    a_rule = a_rule + rule_term(c, s)
                    a_raw = a_raw + raw_term(c, s)
                br, bw = int(bits(a_raw)), int(bits(a_rule))
                if br != bw:
                    differ += 1
                    # only (-0 here, +0 by the rule): redone term by term
                    assert br == 0x80000000 and bw == 0x00000000, (a0, seq)
    assert differ > 0


def test_ternary_fma_form_is_the_rounded_sum():
    # the product f * fl(s/2) is +-s exactly, so fma(f, s/2, a) = fl(a + DQ)
    rng = np.random.default_rng(3)
    s = np.abs(rng.standard_normal(200000).astype(np.float32)) * np.float32(10.0) ** rng.integers(-30, 30, 200000)
    s = s.astype(np.float32)
    s = s[fast_guard(bits(s))]
    for code in range(4):
        t_raw = np.array([raw_term(code, x) for x in s[:2000]], dtype=np.float32)
        t_rule = np.array([rule_term(code, x) for x in s[:2000]], dtype=np.float32)
        if code == 2:
            assert np.all(t_raw == 0.0) and np.all(np.signbit(t_raw))
        else:
            assert np.all(bits(t_raw) == bits(t_rule))


# ---------------------------------------------------------------------- INT2


def code_of(w, j):
    return (w >> (2 * j)) & 3


def v_perm_b32(src0, src1, sel):
    """v_perm_b32 byte select: bytes 0-3 of src1, 4-7 of src0 (selectors
    0-7); 12 gives 0x00 (the only other selector the kernels use)."""
    data = (src0 << 32) | src1
    out = 0
    for i in range(4):
        s = (sel >> (8 * i)) & 0xFF
        if s <= 7:
            byte = (data >> (8 * s)) & 0xFF
        elif s == 12:
            byte = 0
        else:
            raise ValueError(s)
        out |= byte << (8 * i)
    return out


def test_int2_pair_address_bytes():
    rng = np.random.default_rng(4)
    words = [int(w) for w in rng.integers(0, 2**32, 20000, dtype=np.uint64)] + [0, 0xFFFFFFFF, 0xE4E4E4E4]
    for w in words:
        p01 = ((w << 3) & 0xFFFFFFFF) & 0x78787878
        p23 = (w >> 1) & 0x78787878
        for q in range(4):
            assert (p01 >> (8 * q)) & 0xFF == 8 * (code_of(w, 4 * q) + 4 * code_of(w, 4 * q + 1))
            assert (p23 >> (8 * q)) & 0xFF == 8 * (code_of(w, 4 * q + 2) + 4 * code_of(w, 4 * q + 3))


@pytest.mark.parametrize("tbase", [0x0, 0x100, 0x1F00, 0xFF00])
def test_int2_perm_puts_the_byte_over_the_table_base(tbase):
    for byte in range(0, 128, 8):
        for q in range(4):
            sp = byte << (8 * q) | (0x5A5A5A5A & ~(0xFF << (8 * q)))
            assert v_perm_b32(tbase, sp, 0x07060500 | q) == tbase + byte


def test_int2_pair_table_layout():
    # lane l writes float l of the table: code (l & 1 ? l >> 3 : (l >> 1) & 3)
    # entry e = c0 + 4 c1 must hold (d(c0), d(c1)) at floats 2e, 2e + 1
    lane_code = [(l >> 3) if (l & 1) else ((l >> 1) & 3) for l in range(32)]
    for c0 in range(4):
        for c1 in range(4):
            e = c0 + 4 * c1
            assert lane_code[2 * e] == c0 and lane_code[2 * e + 1] == c1
    # the decoded values the table holds are the decoder's: fl(fl(c s) + z)
    rng = np.random.default_rng(5)
    for _ in range(200):
        s, z = np.float32(rng.standard_normal()), np.float32(rng.standard_normal())
        table = [np.float32(np.float32(c) * s) + z for c in lane_code]
        for c0, c1 in itertools.product(range(4), repeat=2):
            e = c0 + 4 * c1
            assert bits(table[2 * e]) == bits(np.float32(np.float32(c0) * s) + z)
            assert bits(table[2 * e + 1]) == bits(np.float32(np.float32(c1) * s) + z)
