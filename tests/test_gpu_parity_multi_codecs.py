"""GPU parity for every encoder's tensor-list form: stochastic uniform,
QSGD, TernGrad, sign (fp32 and bf16 tensors), the shared-scale statistic
and encoder, and top-k each encode a list of tensors, read in place,
exactly as the oracle encodes their concatenation (codes, statistics and
the residual, bit for bit).  Tensor sizes include 0, 1 and sizes that are
not multiples of 4; tensors start at addresses that are not 16-byte
aligned; totals end inside different waves of the last bucket."""
import numpy as np
import pytest

from embedding_communication_codecs_amd import synth
from gpu_util import Out, bits_equal, dev, dev_ef, first_diff, need_gpu, out_f32

pytestmark = pytest.mark.gpu

BUCKETS = [64, 512, 4096, 32768]
CASES = [(b, c) for b in BUCKETS for c in (1, 7, 300)]


@pytest.fixture(scope="module")
def qc():
    return need_gpu()


def sync():
    import torch

    torch.cuda.synchronize()


def random_sizes(rng, count, big):
    pool = [0, 1, 2, 3, 5, 63, 64, 65, 127, 1000, 1021, 4096, 4099]
    sizes = [int(rng.choice(pool)) if rng.random() < 0.7 else int(rng.integers(1, big)) for _ in range(count)]
    if sum(sizes) == 0:
        sizes[0] = 17
    return sizes


def carve(host, dtype="f32", gap=3):
    """One device buffer holding the tensors `gap` elements apart (so most
    start off a 16-byte boundary); returns the buffer and the views."""
    import torch

    sizes = [h.size for h in host]
    total = sum(sizes) + gap * (len(sizes) + 1)
    if dtype == "f32":
        buf = torch.full((total,), -1234.5, dtype=torch.float32, device="cuda")
    else:
        buf = torch.full((total,), -1234.5, dtype=torch.bfloat16, device="cuda")
    views, pos = [], gap
    for h in host:
        v = buf[pos: pos + h.size]
        if dtype == "f32":
            v.copy_(torch.from_numpy(np.ascontiguousarray(h, np.float32)))
        else:
            v.copy_(torch.from_numpy(np.ascontiguousarray(h).view(np.int16)).cuda().view(torch.bfloat16))
        views.append(v)
        pos += h.size + gap
    return buf, views


def inputs(count, bucket, seed, tail=None):
    rng = np.random.default_rng(seed)
    sizes = random_sizes(rng, count, 3 * bucket)
    if tail is not None:  # total = 2 buckets + tail, the last tensor absorbing the difference
        sizes[-1] += max(0, 2 * bucket + tail - sum(sizes))
        while sum(sizes) > 2 * bucket + tail:
            k = int(np.argmax(sizes))
            sizes[k] -= min(sizes[k], sum(sizes) - (2 * bucket + tail))
    host = [synth.host_outlier_grad(max(s, 1), 1e-3, 0.01, 100.0, seed=seed + k)[:s] for k, s in enumerate(sizes)]
    return host


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("bucket,count", CASES)
def test_stochastic_uniform_multi(qc, ora, bucket, count, bits):
    host = inputs(count, bucket, 100 + count + bits)
    flat = ora.concat(host)
    n = flat.size
    nb = qc.nbuckets(n, bucket)
    ef_h = synth.host_normal(n, 1e-4, seed=count)
    ef_d = dev_ef(ef_h)
    _, views = carve(host)
    t = qc.TensorTable(views)
    codes = Out(qc.payload_bytes(qc.QC_UNIFORM, n, bucket, bits))
    scale, zero = out_f32(nb), out_f32(nb)
    qc.qc_encode_uniform_stochastic_multi(t.xs, t.offsets, t.seg_first, t.ntensors, n, ef_d.t, bucket, bits,
                                          0x53544F43, 4 * count, codes.t, scale.t, zero.t)
    sync()
    p, s, z = ora.encode_uniform_stochastic(flat, ef_h, bucket, bits, 0x53544F43, 4 * count)
    assert bits_equal(codes.host(), p), first_diff(codes.host(), p)
    assert bits_equal(scale.f32(), s) and bits_equal(zero.f32(), z)
    assert bits_equal(ef_d.f32(), ef_h), first_diff(ef_d.f32(), ef_h)


@pytest.mark.parametrize("bucket,count", CASES)
def test_qsgd_and_ternary_multi(qc, ora, bucket, count):
    host = inputs(count, bucket, 200 + count)
    flat = ora.concat(host)
    n = flat.size
    nb = qc.nbuckets(n, bucket)
    _, views = carve(host)
    t = qc.TensorTable(views)
    ef_h = synth.host_normal(n, 1e-5, seed=count)
    ef_d = dev_ef(ef_h)
    words, norm = Out(qc.payload_bytes(qc.QC_QSGD, n, bucket, 16)), out_f32(nb)
    qc.qc_encode_qsgd_multi(t.xs, t.offsets, t.seg_first, t.ntensors, n, ef_d.t, bucket, 16, 0x5153474400000001,
                            8, words.t, norm.t)
    sync()
    p, nr = ora.encode_qsgd(flat, ef_h, bucket, 0x5153474400000001, 8)
    assert bits_equal(words.host(), p), first_diff(words.host(), p)
    assert bits_equal(norm.f32(), nr) and bits_equal(ef_d.f32(), ef_h), first_diff(ef_d.f32(), ef_h)

    ef_h = synth.host_normal(n, 1e-5, seed=count + 1)
    ef_d = dev_ef(ef_h)
    words, scale = Out(qc.payload_bytes(qc.QC_TERNARY, n, bucket, 2)), out_f32(nb)
    qc.qc_encode_ternary_multi(t.xs, t.offsets, t.seg_first, t.ntensors, n, ef_d.t, bucket, 0x5445524E, 0,
                               words.t, scale.t)
    sync()
    p, s = ora.encode_ternary(flat, ef_h, bucket, 0x5445524E, 0)
    assert bits_equal(words.host(), p) and bits_equal(scale.f32(), s), first_diff(words.host(), p)
    assert bits_equal(ef_d.f32(), ef_h), first_diff(ef_d.f32(), ef_h)


@pytest.mark.parametrize("bucket,count", CASES + [(65536, 5), (16384, 40)])
def test_topk_multi(qc, ora, bucket, count):
    host = inputs(count, bucket, 700 + count)
    flat = ora.concat(host)
    n = flat.size
    nb = qc.nbuckets(n, bucket)
    _, views = carve(host)
    t = qc.TensorTable(views)
    for k in sorted({1, 5, max(1, bucket // 100), bucket}):
        ef_h = synth.host_normal(n, 1e-4, seed=count + k)
        ef_d = dev_ef(ef_h)
        vals, idx = out_f32(nb * k), Out(4 * nb * k)
        qc.qc_encode_topk_multi(t.xs, t.offsets, t.seg_first, t.ntensors, n, ef_d.t, bucket, k, vals.t, idx.t)
        sync()
        pv, pi = ora.encode_topk(flat, ef_h, bucket, k)
        assert bits_equal(idx.host().view(np.uint32), pi), (k, first_diff(idx.host().view(np.uint32), pi))
        assert bits_equal(vals.f32(), pv), (k, first_diff(vals.f32(), pv))
        assert bits_equal(ef_d.f32(), ef_h), (k, first_diff(ef_d.f32(), ef_h))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bucket,count", CASES)
def test_sign_multi(qc, ora, bucket, count, dtype):
    host = inputs(count, bucket, 300 + count)
    if dtype == "bf16":
        host = [synth.host_bf16_bits(h) for h in host]
    flat = np.concatenate(host) if host else host
    n = flat.size
    nb = qc.nbuckets(n, bucket)
    _, views = carve(host, dtype)
    t = qc.TensorTable(views)
    ef_h = synth.host_normal(n, 1e-4, seed=count)
    ef_d = dev_ef(ef_h)
    words, scale = Out(qc.payload_bytes(qc.QC_SIGN, n, bucket, 1)), out_f32(nb)
    xtype = qc.QC_BF16 if dtype == "bf16" else qc.QC_F32
    qc.qc_encode_sign_multi(t.xs, xtype, t.offsets, t.seg_first, t.ntensors, n, ef_d.t, bucket, words.t, scale.t)
    sync()
    p, s = ora.encode_sign(flat, ef_h, bucket)
    assert bits_equal(words.host(), p), first_diff(words.host(), p)
    assert bits_equal(scale.f32(), s), first_diff(scale.f32(), s)
    assert bits_equal(ef_d.f32(), ef_h), first_diff(ef_d.f32(), ef_h)


@pytest.mark.parametrize("bucket,count", CASES)
def test_shared_scale_multi(qc, ora, bucket, count):
    host = inputs(count, bucket, 400 + count)
    flat = ora.concat(host)
    n = flat.size
    nb = qc.nbuckets(n, bucket)
    _, views = carve(host)
    t = qc.TensorTable(views)
    ef_h = synth.host_normal(n, 1e-4, seed=count)
    amax = out_f32(nb)
    qc.qc_bucket_absmax_multi(t.xs, t.offsets, t.seg_first, t.ntensors, n, dev(ef_h), bucket, amax.t)
    sync()
    want = ora.bucket_absmax(flat, ef_h, bucket)
    assert bits_equal(amax.f32(), want), first_diff(amax.f32(), want)
    ef_d = dev_ef(ef_h)
    codes, scale = Out(qc.payload_bytes(qc.QC_INT8_SHARED, n, bucket, 8)), out_f32(nb)
    qc.qc_encode_int8_shared_multi(t.xs, t.offsets, t.seg_first, t.ntensors, n, ef_d.t, bucket, dev(want), codes.t,
                                   scale.t)
    sync()
    p, s = ora.encode_int8_shared(flat, ef_h, bucket, want)
    assert bits_equal(codes.host(), p) and bits_equal(scale.f32(), s), first_diff(codes.host(), p)
    assert bits_equal(ef_d.f32(), ef_h), first_diff(ef_d.f32(), ef_h)


# buckets of 4,096 hold 512 elements per wave over 8 waves, buckets of
# 32,768 hold 2,048 per wave over 16 (bf16: twice as many per wave)
TAILS = [(4096, t) for t in (5, 3 * 512 + 1, 4095)] + [(32768, t) for t in (3, 9 * 2048 + 7, 32767)]


@pytest.mark.parametrize("bucket,tail", TAILS)
def test_list_tails_inside_every_wave(qc, ora, bucket, tail):
    """Every list encoder on a list whose total ends inside the first, a
    middle and the last wave of its last bucket."""
    host = inputs(9, bucket, 500 + tail, tail=tail)
    flat = ora.concat(host)
    n = flat.size
    assert n == 2 * bucket + tail
    nb = qc.nbuckets(n, bucket)
    _, views = carve(host)
    t = qc.TensorTable(views)
    L = (t.xs, t.offsets, t.seg_first, t.ntensors, n)

    ef_h = synth.host_normal(n, 1e-4, seed=1)
    ef_d = dev_ef(ef_h)
    codes, scale, zero = Out(qc.payload_bytes(qc.QC_UNIFORM, n, bucket, 4)), out_f32(nb), out_f32(nb)
    qc.qc_encode_uniform_stochastic_multi(*L, ef_d.t, bucket, 4, 77, 0, codes.t, scale.t, zero.t)
    sync()
    p, s, z = ora.encode_uniform_stochastic(flat, ef_h, bucket, 4, 77, 0)
    assert bits_equal(codes.host(), p) and bits_equal(ef_d.f32(), ef_h), "stochastic uniform"

    ef_h = synth.host_normal(n, 1e-4, seed=2)
    ef_d = dev_ef(ef_h)
    words, norm = Out(qc.payload_bytes(qc.QC_QSGD, n, bucket, 16)), out_f32(nb)
    qc.qc_encode_qsgd_multi(*L, ef_d.t, bucket, 16, 5, 0, words.t, norm.t)
    sync()
    p, nr = ora.encode_qsgd(flat, ef_h, bucket, 5, 0)
    assert bits_equal(words.host(), p) and bits_equal(norm.f32(), nr) and bits_equal(ef_d.f32(), ef_h), "qsgd"

    ef_h = synth.host_normal(n, 1e-4, seed=3)
    ef_d = dev_ef(ef_h)
    words, scale = Out(qc.payload_bytes(qc.QC_SIGN, n, bucket, 1)), out_f32(nb)
    qc.qc_encode_sign_multi(t.xs, qc.QC_F32, t.offsets, t.seg_first, t.ntensors, n, ef_d.t, bucket, words.t, scale.t)
    sync()
    p, s = ora.encode_sign(flat, ef_h, bucket)
    assert bits_equal(words.host(), p) and bits_equal(scale.f32(), s) and bits_equal(ef_d.f32(), ef_h), "sign"

    hb = [synth.host_bf16_bits(h) for h in host]
    _, bviews = carve(hb, "bf16")
    tb = qc.TensorTable(bviews)
    ef_h = synth.host_normal(n, 1e-4, seed=4)
    ef_d = dev_ef(ef_h)
    words, scale = Out(qc.payload_bytes(qc.QC_SIGN, n, bucket, 1)), out_f32(nb)
    qc.qc_encode_sign_multi(tb.xs, qc.QC_BF16, tb.offsets, tb.seg_first, tb.ntensors, n, ef_d.t, bucket, words.t,
                            scale.t)
    sync()
    p, s = ora.encode_sign(np.concatenate(hb), ef_h, bucket)
    assert bits_equal(words.host(), p) and bits_equal(scale.f32(), s) and bits_equal(ef_d.f32(), ef_h), "sign bf16"

    ef_h = synth.host_normal(n, 1e-4, seed=5)
    ef_d = dev_ef(ef_h)
    words, scale = Out(qc.payload_bytes(qc.QC_TERNARY, n, bucket, 2)), out_f32(nb)
    qc.qc_encode_ternary_multi(*L, ef_d.t, bucket, 9, 4, words.t, scale.t)
    sync()
    p, s = ora.encode_ternary(flat, ef_h, bucket, 9, 4)
    assert bits_equal(words.host(), p) and bits_equal(scale.f32(), s) and bits_equal(ef_d.f32(), ef_h), "ternary"


@pytest.mark.skip(reason="not built: at buckets of 65,536 the tensor-list encoders need more registers than a "
                         "lane has and spill to scratch memory; spilled builds of the 65,536-element encoders "
                         "gave results that differ from their source's (the same source matched the oracle on "
                         "the CPU), so the list entry points refuse that size (QC_ERR_UNSUPPORTED)")
def test_list_bucket_65536(qc, ora):
    host = inputs(1, 65536, 600)
    _, views = carve(host)
    t = qc.TensorTable(views)
    n = t.n
    codes, scale, zero = Out(qc.payload_bytes(qc.QC_UNIFORM, n, 65536, 8)), out_f32(1), out_f32(1)
    qc.qc_encode_uniform_multi(t.xs, t.offsets, t.seg_first, t.ntensors, n, None, 65536, 8, codes.t, scale.t,
                               zero.t)
    sync()
    p, s, z = ora.encode_uniform(ora.concat(host), None, 65536, 8)
    assert bits_equal(codes.host(), p)
