"""GPU parity for the largest buckets, 16,384, 32,768 and 65,536 elements,
which spread one bucket over 8 or 16 waves (up to 16 chunks per lane):
every encoder with error feedback and its decode, and the worker sums with
fused requantization, on inputs whose last bucket ends inside the first, a
middle and the last wave of the bucket.  Results must equal the oracle's
bit for bit."""
import numpy as np
import pytest

from embedding_communication_codecs_amd import synth
from gpu_util import Out, bits_equal, dev, dev_ef, first_diff, need_gpu, out_f32

pytestmark = pytest.mark.gpu

# (bucket, elements per wave of the fp32 encoders' layout)
SIZES = [(16384, 2048), (32768, 2048), (65536, 4096)]
CASES = [(b, t) for b, w in SIZES for t in (5, 3 * w + 1, b - 3)]
IDS = [f"B{b}-tail{t}" for b, t in CASES]


@pytest.fixture(scope="module")
def qc():
    return need_gpu()


def sync():
    import torch

    torch.cuda.synchronize()


def decoded(qc, fmt, codes, scale, zero, n, bucket, bits):
    out = out_f32(n)
    qc.qc_decode(fmt, codes.t, scale.t, None if zero is None else zero.t, n, bucket, bits, out.t)
    sync()
    return out.f32()


@pytest.mark.parametrize("bucket,tail", CASES, ids=IDS)
def test_uniform_large_buckets(qc, ora, bucket, tail):
    n = 2 * bucket + tail
    g = synth.host_outlier_grad(n, 1e-3, 0.01, 100.0, seed=bucket + tail)
    nb = qc.nbuckets(n, bucket)
    for bits in (8, 4, 2):
        for stoch in (False, True):
            ef_h = synth.host_normal(n, 1e-4, seed=bits + tail)
            ef_d = dev_ef(ef_h)
            codes = Out(qc.payload_bytes(qc.QC_UNIFORM, n, bucket, bits))
            scale, zero = out_f32(nb), out_f32(nb)
            if stoch:
                qc.qc_encode_uniform_stochastic(dev(g), ef_d.t, n, bucket, bits, 0x53544F43, 4 * tail, codes.t,
                                                scale.t, zero.t)
                p, s, z = ora.encode_uniform_stochastic(g, ef_h, bucket, bits, 0x53544F43, 4 * tail)
            else:
                qc.qc_encode_uniform(dev(g), ef_d.t, n, bucket, bits, codes.t, scale.t, zero.t)
                p, s, z = ora.encode_uniform(g, ef_h, bucket, bits)
            sync()
            assert bits_equal(codes.host(), p), (bits, stoch, first_diff(codes.host(), p))
            assert bits_equal(scale.f32(), s) and bits_equal(zero.f32(), z), (bits, stoch)
            assert bits_equal(ef_d.f32(), ef_h), (bits, stoch, first_diff(ef_d.f32(), ef_h))
            want = ora.decode_uniform(p, s, z, n, bucket, bits)
            got = decoded(qc, qc.QC_UNIFORM, codes, scale, zero, n, bucket, bits)
            assert bits_equal(got, want), (bits, stoch, first_diff(got, want))


@pytest.mark.parametrize("bucket,tail", CASES, ids=IDS)
def test_qsgd_ternary_large_buckets(qc, ora, bucket, tail):
    n = 2 * bucket + tail
    g = synth.host_laplace(n, 1e-4, seed=bucket + tail)
    nb = qc.nbuckets(n, bucket)
    ef_h = synth.host_normal(n, 1e-5, seed=tail)
    ef_d = dev_ef(ef_h)
    words = Out(qc.payload_bytes(qc.QC_QSGD, n, bucket, 16))
    norm = out_f32(nb)
    qc.qc_encode_qsgd(dev(g), ef_d.t, n, bucket, 16, 0x5153474400000001, 8, words.t, norm.t)
    sync()
    p, nr = ora.encode_qsgd(g, ef_h, bucket, 0x5153474400000001, 8)
    assert bits_equal(words.host(), p), first_diff(words.host(), p)
    assert bits_equal(norm.f32(), nr) and bits_equal(ef_d.f32(), ef_h), first_diff(ef_d.f32(), ef_h)
    got = decoded(qc, qc.QC_QSGD, words, norm, None, n, bucket, 16)
    want = ora.decode_qsgd(p, nr, n, bucket)
    assert bits_equal(got, want), first_diff(got, want)

    ef_h = synth.host_normal(n, 1e-5, seed=tail + 1)
    ef_d = dev_ef(ef_h)
    words = Out(qc.payload_bytes(qc.QC_TERNARY, n, bucket, 2))
    scale = out_f32(nb)
    qc.qc_encode_ternary(dev(g), ef_d.t, n, bucket, 0x5445524E, 0, words.t, scale.t)
    sync()
    p, s = ora.encode_ternary(g, ef_h, bucket, 0x5445524E, 0)
    assert bits_equal(words.host(), p) and bits_equal(scale.f32(), s), first_diff(words.host(), p)
    assert bits_equal(ef_d.f32(), ef_h), first_diff(ef_d.f32(), ef_h)
    got = decoded(qc, qc.QC_TERNARY, words, scale, None, n, bucket, 2)
    assert bits_equal(got, ora.decode_ternary(p, s, n, bucket))


@pytest.mark.parametrize("bucket,tail", CASES, ids=IDS)
def test_sign_and_shared_large_buckets(qc, ora, bucket, tail):
    n = 2 * bucket + tail
    g = synth.host_normal(n, 1e-3, seed=bucket + tail + 1)
    nb = qc.nbuckets(n, bucket)
    for x in (g, synth.host_bf16_bits(g)):
        ef_h = synth.host_normal(n, 1e-4, seed=tail + 2)
        ef_d = dev_ef(ef_h)
        words = Out(qc.payload_bytes(qc.QC_SIGN, n, bucket, 1))
        scale = out_f32(nb)
        xt = qc.QC_BF16 if x.dtype == np.uint16 else qc.QC_F32
        qc.qc_encode_sign(dev(x), xt, ef_d.t, n, bucket, words.t, scale.t)
        sync()
        p, s = ora.encode_sign(x, ef_h, bucket)
        assert bits_equal(words.host(), p), (x.dtype, first_diff(words.host(), p))
        assert bits_equal(scale.f32(), s), (x.dtype, first_diff(scale.f32(), s))
        assert bits_equal(ef_d.f32(), ef_h), (x.dtype, first_diff(ef_d.f32(), ef_h))
        got = decoded(qc, qc.QC_SIGN, words, scale, None, n, bucket, 1)
        assert bits_equal(got, ora.decode_sign(p, s, n, bucket)), x.dtype

    x = synth.host_outlier_grad(n, 1e-3, 0.01, 100.0, seed=tail + 3)
    ef_h = synth.host_normal(n, 1e-4, seed=tail + 4)
    amax = out_f32(nb)
    qc.qc_bucket_absmax(dev(x), dev(ef_h), n, bucket, amax.t)
    sync()
    want_amax = ora.bucket_absmax(x, ef_h, bucket)
    assert bits_equal(amax.f32(), want_amax), first_diff(amax.f32(), want_amax)
    ef_d = dev_ef(ef_h)
    codes = Out(qc.payload_bytes(qc.QC_INT8_SHARED, n, bucket, 8))
    scale = out_f32(nb)
    qc.qc_encode_int8_shared(dev(x), ef_d.t, n, bucket, dev(want_amax), codes.t, scale.t)
    sync()
    p, s = ora.encode_int8_shared(x, ef_h, bucket, want_amax)
    assert bits_equal(codes.host(), p) and bits_equal(scale.f32(), s), first_diff(codes.host(), p)
    assert bits_equal(ef_d.f32(), ef_h), first_diff(ef_d.f32(), ef_h)


def payloads(ora, fmt, m, n, group, seed):
    parts, sc, ze = [], [], []
    for w in range(m):
        g = synth.host_outlier_grad(n, 1e-3, 0.01, 100.0, seed=seed + w)
        if fmt in ("u8", "u4", "u2"):
            p, s, z = ora.encode_uniform(g, None, group, {"u8": 8, "u4": 4, "u2": 2}[fmt])
            ze.append(z)
        elif fmt == "qsgd":
            p, s = ora.encode_qsgd(g, None, group, seed + w, 0)
        elif fmt == "ter":
            p, s = ora.encode_ternary(g, None, group, seed + w, 0)
        else:
            p, s = ora.encode_sign(g, None, group)
        parts.append(p)
        sc.append(s)
    return np.concatenate(parts), np.concatenate(sc), (np.concatenate(ze) if ze else None)


# (C-ABI format, bits, oracle format, oracle bits)
ACC_FMT = {"u8": (0, 8, 0, 8), "u4": (0, 4, 0, 4), "u2": (0, 2, 0, 2), "qsgd": (2, 16, 2, 4),
           "sign": (3, 1, 3, 1), "ter": (4, 2, 4, 2)}


@pytest.mark.parametrize("fmt", list(ACC_FMT))
@pytest.mark.parametrize("group,tail", [(16384, 2 * 4096 + 7), (32768, 5), (65536, 65536 - 21)])
def test_worker_sums_large_groups(qc, ora, fmt, group, tail):
    """Worker sums in worker order (bit-exact), and for the uniform formats
    the fused requantization of the sum.  The sums hold a bucket as W waves
    of 4,096 elements (W = group / 4096), so the tails end inside wave 2 of
    4, wave 0 of 8 and the last of 16."""
    m, n = 5, group + tail
    code, bits, ofmt, obits = ACC_FMT[fmt]
    p, s, z = payloads(ora, fmt, m, n, group, seed=7100 + group % 1000)
    want = ora.dequant_accumulate(ofmt, p, s, z, m, n, group, obits)
    acc = out_f32(n)
    nb = qc.nbuckets(n, group)
    rq = rqs = rqz = None
    if fmt in ("u8", "u4", "u2"):
        rq = Out(qc.payload_bytes(qc.QC_UNIFORM, n, group, bits))
        rqs, rqz = out_f32(nb), out_f32(nb)
    qc.qc_dequant_accumulate(code, dev(p), dev(s), None if z is None else dev(z), m, n, group, bits, acc.t, False,
                             None if rq is None else rq.t, None if rqs is None else rqs.t,
                             None if rqz is None else rqz.t)
    sync()
    assert bits_equal(acc.f32(), want), first_diff(acc.f32(), want)
    if rq is not None:
        pq, sq, zq = ora.encode_uniform(want, None, group, bits)
        assert bits_equal(rq.host(), pq), first_diff(rq.host(), pq)
        assert bits_equal(rqs.f32(), sq) and bits_equal(rqz.f32(), zq)
