"""GPU parity at the edges of a division shortcut: the QSGD encoder
computes |v| / d from the bucket's reciprocal and divides only where that
is not exact (d or 1/d outside the normal range, |v| below 2^-102, a
quotient below 2^-100).  Buckets here put elements on both sides of each of
those limits, in the same wave as ordinary ones.  The same inputs, with
scales just inside and just outside the normal range and negative or
infinite shared scales, also run through the uniform, stochastic uniform,
TernGrad and shared-scale INT8 encoders, which divide element by element.
Codes, scales and residuals must match the oracle bit for bit."""
import numpy as np
import pytest

from embedding_communication_codecs_amd import synth
from gpu_util import Out, bits_equal, dev, dev_ef, first_diff, need_gpu, out_f32

pytestmark = pytest.mark.gpu

B = 64
TWO126 = np.float32(2.0 ** 126)


@pytest.fixture(scope="module")
def qc():
    return need_gpu()


def sync():
    import torch

    torch.cuda.synchronize()


def bucket(head, fill, seed):
    """head values first, the rest of a 64-element bucket from `fill`."""
    rng = np.random.default_rng(seed)
    rest = np.asarray(fill(rng, B - len(head)), np.float32)
    return np.concatenate([np.asarray(head, np.float32), rest])


def tiny_mix(rng, k):
    # below 2^-102, just above it, and ordinary magnitudes, both signs
    vals = np.array([1e-35, 3e-36, 2.0 ** -103, 2.0 ** -102, 2.0 ** -101, 1e-29, 1e-20, 1e-10, 0.0, -0.0], np.float32)
    out = vals[rng.integers(0, vals.size, k)] * np.where(rng.random(k) < 0.5, -1, 1)
    return out.astype(np.float32)


def rows_general():
    return np.concatenate([
        bucket([1000.0, -1000.0], tiny_mix, 1),                     # quotients far below 2^-100
        bucket([1e30, 0.0], tiny_mix, 2),                            # huge scale, tiny elements
        bucket([2.0 ** -120, -(2.0 ** -121)], lambda r, k: r.standard_normal(k) * 2.0 ** -124, 3),
        bucket([1.0], lambda r, k: r.standard_normal(k), 4),         # ordinary
        bucket([1e-3, -1e-3], lambda r, k: r.laplace(0, 1e-4, k), 5),
    ]).astype(np.float32)


def rows_scale_limits(levels):
    """Buckets whose scale (range / levels) lands just below, at and just
    above 2^126, and at 2^-126."""
    out = []
    for f in (0.999, 1.0, 1.001):
        with np.errstate(over="ignore"):
            span = np.float32(TWO126 * np.float32(levels) * np.float32(f))
        if not np.isfinite(span):
            continue
        out.append(bucket([0.0, span], lambda r, k: r.random(k) * span, 10))
    small = np.float32(2.0 ** -126) * np.float32(levels)
    out.append(bucket([0.0, small], lambda r, k: r.random(k).astype(np.float32) * small, 11))
    return np.concatenate(out).astype(np.float32)


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("stochastic", [False, True])
def test_uniform_quotient_edges(qc, ora, bits, stochastic):
    x = np.concatenate([rows_general(), rows_scale_limits((1 << bits) - 1)])
    n = x.size
    ef_h = synth.host_normal(n, 1e-30, seed=21)
    ef_d = dev_ef(ef_h)
    nb = qc.nbuckets(n, B)
    codes = Out(qc.payload_bytes(qc.QC_UNIFORM, n, B, bits))
    scale, zero = out_f32(nb), out_f32(nb)
    if stochastic:
        qc.qc_encode_uniform_stochastic(dev(x), ef_d.t, n, B, bits, 0xABCDEF, 16, codes.t, scale.t, zero.t)
        p, s, z = ora.encode_uniform_stochastic(x, ef_h, B, bits, 0xABCDEF, 16)
    else:
        qc.qc_encode_uniform(dev(x), ef_d.t, n, B, bits, codes.t, scale.t, zero.t)
        p, s, z = ora.encode_uniform(x, ef_h, B, bits)
    sync()
    assert bits_equal(codes.host(), p), first_diff(codes.host(), p)
    assert bits_equal(scale.f32(), s) and bits_equal(zero.f32(), z)
    assert bits_equal(ef_d.f32(), ef_h), first_diff(ef_d.f32(), ef_h)


@pytest.mark.parametrize("bucket", [64, 512, 4096, 65536])
def test_qsgd_quotient_edges(qc, ora, bucket):
    # the 64-element rows tiled over larger buckets (a ragged last one),
    # without the row whose squares overflow (it would make every norm inf)
    x = rows_general()
    if bucket > B:
        x = np.resize(np.concatenate([x[:B], x[2 * B:]]), 2 * bucket + 37)
    n = x.size
    for step, seed in enumerate((7, 8)):
        ef_h = synth.host_normal(n, 1e-31, seed=30 + step)
        ef_d = dev_ef(ef_h)
        words = Out(qc.payload_bytes(qc.QC_QSGD, n, bucket, 16))
        norm = out_f32(qc.nbuckets(n, bucket))
        qc.qc_encode_qsgd(dev(x), ef_d.t, n, bucket, 16, seed, 0, words.t, norm.t)
        sync()
        p, nr = ora.encode_qsgd(x, ef_h, bucket, seed, 0)
        assert bits_equal(words.host(), p), first_diff(words.host(), p)
        assert bits_equal(norm.f32(), nr) and bits_equal(ef_d.f32(), ef_h)


def test_ternary_quotient_edges(qc, ora):
    x = np.concatenate([rows_general(), rows_scale_limits(1)])
    n = x.size
    ef_h = synth.host_normal(n, 1e-31, seed=41)
    ef_d = dev_ef(ef_h)
    words = Out(qc.payload_bytes(qc.QC_TERNARY, n, B, 2))
    scale = out_f32(qc.nbuckets(n, B))
    qc.qc_encode_ternary(dev(x), ef_d.t, n, B, 0x7E57, 0, words.t, scale.t)
    sync()
    p, s = ora.encode_ternary(x, ef_h, B, 0x7E57, 0)
    assert bits_equal(words.host(), p), first_diff(words.host(), p)
    assert bits_equal(scale.f32(), s) and bits_equal(ef_d.f32(), ef_h)


def test_shared_int8_quotient_edges(qc, ora):
    amaxes = np.array([1.0, -1.0, 127 * 2.0 ** -126, 127 * 2.0 ** -126 * 0.999, 127 * 2.0 ** -126 * 1.001,
                       3e38, np.inf, 0.0, -0.0, 1e30, 2.5], np.float32)
    rng = np.random.default_rng(50)
    rows = []
    for i, a in enumerate(amaxes):
        mag = np.float32(1.0) if not np.isfinite(a) or a == 0 else abs(a)
        fill = rng.standard_normal(B // 2) * mag * 0.5
        rows.append(np.concatenate([tiny_mix(rng, B // 2), fill]).astype(np.float32))
    x = np.concatenate(rows).astype(np.float32)
    n = x.size
    ef_h = synth.host_normal(n, 1e-31, seed=51)
    ef_d = dev_ef(ef_h)
    codes = Out(qc.payload_bytes(qc.QC_INT8_SHARED, n, B, 8))
    scale = out_f32(qc.nbuckets(n, B))
    qc.qc_encode_int8_shared(dev(x), ef_d.t, n, B, dev(amaxes), codes.t, scale.t)
    sync()
    p, s = ora.encode_int8_shared(x, ef_h, B, amaxes)
    assert bits_equal(codes.host(), p), first_diff(codes.host(), p)
    ok = ~(np.isnan(scale.f32()) & np.isnan(s))
    assert bits_equal(scale.f32()[ok], s[ok])
    eg, ew = ef_d.f32(), ef_h
    both_nan = np.isnan(eg) & np.isnan(ew)
    assert bits_equal(eg[~both_nan], ew[~both_nan]), first_diff(eg, ew)
