"""GPU parity for top-k sparsification: the encoder (both selection paths:
the candidate path for small k and the radix select; pairs in index order,
error feedback), the decoder (scatter into a dense vector)
and the sum of several workers' sparse payloads, each called through the C
ABI and compared bit for bit with the CPU oracle on the same seeded inputs:
every bucket size (16,384 to 65,536 through the streaming encoder and the
tiled decoder and sums), k from 1 to the whole bucket, short last buckets,
many equal magnitudes (ties go to the smaller index), signed zeros."""
import numpy as np
import pytest

from embedding_communication_codecs_amd import synth
from gpu_util import Out, bits_equal, dev, dev_ef, first_diff, need_gpu, out_f32

pytestmark = pytest.mark.gpu

BUCKETS = [64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384, 32768, 65536]


@pytest.fixture(scope="module")
def qc():
    return need_gpu()


def sync():
    import torch

    torch.cuda.synchronize()


def run_topk(qc, x, ef, bucket, k):
    import torch

    n = x.size
    slots = qc.nbuckets(n, bucket) * k
    vals = out_f32(slots)
    idx = Out(4 * slots, torch.int32)
    qc.qc_encode_topk(dev(x), None if ef is None else ef.t, n, bucket, k, vals.t, idx.t)
    sync()
    return vals, idx


def ks_for(bucket):
    return sorted({1, 3, max(1, bucket // 1000), bucket // 16, bucket // 2 + 1, bucket})


def gradient_like(n, seed, ties=False):
    x = synth.host_outlier_grad(n, 1e-3, 0.01, 100.0, seed=seed)
    if ties:  # few distinct magnitudes: the threshold is shared by many
        x = (np.round(x / 1e-3) * 1e-3).astype(np.float32)
        x[::7] = -0.0
        x[3::11] = 0.0
    return x


@pytest.mark.parametrize("bucket", BUCKETS)
def test_topk_encode_parity_ef_steps(qc, ora, bucket):
    n = 3 * bucket + 37
    for k in ks_for(bucket):
        ef_h = np.zeros(n, np.float32)
        ef_d = dev_ef(ef_h)
        for step in range(2):
            g = gradient_like(n, seed=bucket + 17 * k + step, ties=(k % 2 == 1))
            vals, idx = run_topk(qc, g, ef_d, bucket, k)
            pv, pi = ora.encode_topk(g, ef_h, bucket, k)
            assert bits_equal(idx.host().view(np.uint32), pi), (k, step, first_diff(idx.host().view(np.uint32), pi))
            assert bits_equal(vals.f32(), pv), (k, step, first_diff(vals.f32(), pv))
            assert bits_equal(ef_d.f32(), ef_h), (k, step, first_diff(ef_d.f32(), ef_h))


@pytest.mark.parametrize("n", [1, 5, 63, 64, 65, 1000, 4096 * 3 + 3])
@pytest.mark.parametrize("k", [1, 2, 40, 64])
def test_topk_ragged_no_ef(qc, ora, n, k):
    x = gradient_like(n, seed=n * 3 + k, ties=True)
    vals, idx = run_topk(qc, x, None, 64, k)
    pv, pi = ora.encode_topk(x, None, 64, k)
    assert bits_equal(idx.host().view(np.uint32), pi)
    assert bits_equal(vals.f32(), pv)


def test_topk_special_magnitudes(qc, ora):
    """Equal magnitudes of both signs, signed zeros, subnormals, the largest
    finite values: keys differing only in their lowest bits."""
    B = 256
    base = np.float32(1.0)
    rows = [
        np.where(np.arange(B) % 2 == 0, 1.5, -1.5).astype(np.float32),
        np.array([-0.0, 0.0] * (B // 2), np.float32),
        np.array([1e-45, -1e-45, 3e-39, -2e-39] * (B // 4), np.float32),
        np.array([3.4e38, -3.4e38] + [1.0] * (B - 2), np.float32),
        (base + np.arange(B, dtype=np.float32) * np.float32(2 ** -23)).astype(np.float32)[::-1].copy(),
    ]
    x = np.concatenate(rows)
    for k in (1, 2, 5, 128, 255):
        ef_h = np.zeros(x.size, np.float32)
        ef_d = dev_ef(ef_h)
        vals, idx = run_topk(qc, x, ef_d, B, k)
        pv, pi = ora.encode_topk(x, ef_h, B, k)
        assert bits_equal(idx.host().view(np.uint32), pi), k
        assert bits_equal(vals.f32(), pv), k
        assert bits_equal(ef_d.f32(), ef_h), k


@pytest.mark.parametrize("k", [1, 8, 32, 33])
def test_topk_many_candidates_fall_back(qc, ora, k):
    """Small k, but every magnitude equal (or nearly): more elements pass the
    candidate bound than one wave holds, so the radix select decides."""
    B = 4096
    x = np.where(np.arange(3 * B) % 3 == 0, 2.0, -2.0).astype(np.float32)
    x[5000:5100] = np.float32(2.0000002)  # a few larger keys in bucket 1
    ef_h = np.zeros(x.size, np.float32)
    ef_d = dev_ef(ef_h)
    vals, idx = run_topk(qc, x, ef_d, B, k)
    pv, pi = ora.encode_topk(x, ef_h, B, k)
    assert bits_equal(idx.host().view(np.uint32), pi)
    assert bits_equal(vals.f32(), pv)
    assert bits_equal(ef_d.f32(), ef_h)


@pytest.mark.parametrize("bucket,k", [(64, 1), (64, 64), (1024, 10), (8192, 8), (8192, 5000), (16384, 100),
                                      (32768, 32768), (65536, 3000)])
def test_topk_decode(qc, ora, bucket, k):
    n = 2 * bucket + 13
    x = gradient_like(n, seed=k, ties=True)
    pv, pi = ora.encode_topk(x, None, bucket, k)
    out = out_f32(n)
    qc.qc_decode_topk(dev(pv), dev(pi.view(np.int32)), n, bucket, k, out.t)
    sync()
    want = ora.decode_topk(pv, pi, n, bucket, k)
    assert bits_equal(out.f32(), want), first_diff(out.f32(), want)


@pytest.mark.parametrize("bucket,k", [(64, 3), (1024, 10), (8192, 8), (4096, 2048), (32768, 8), (65536, 300)])
@pytest.mark.parametrize("m", [1, 3, 64])
def test_topk_accumulate(qc, ora, bucket, k, m):
    n = 2 * bucket + 13
    vals, idxs = [], []
    for w in range(m):
        v, i = ora.encode_topk(gradient_like(n, seed=100 * w + k), None, bucket, k)
        vals.append(v)
        idxs.append(i)
    V, I = np.concatenate(vals), np.concatenate(idxs)
    acc = out_f32(n)
    qc.qc_topk_accumulate(dev(V), dev(I.view(np.int32)), m, n, bucket, k, acc.t, False)
    sync()
    want = ora.topk_accumulate(V, I, m, n, bucket, k)
    assert bits_equal(acc.f32(), want), first_diff(acc.f32(), want)
    start = synth.host_normal(n, 1e-3, seed=5)
    start[::9] = -0.0
    acc.t.copy_(dev(start))
    qc.qc_topk_accumulate(dev(V), dev(I.view(np.int32)), m, n, bucket, k, acc.t, True)
    sync()
    want2 = ora.topk_accumulate(V, I, m, n, bucket, k, acc=start)
    assert bits_equal(acc.f32(), want2), first_diff(acc.f32(), want2)


def test_topk_random_shapes(qc, ora):
    rng = np.random.default_rng(404)
    for trial in range(40):
        bucket = int(2 ** rng.integers(6, 17))
        n = int(rng.integers(1, 4 * bucket))
        k = int(rng.integers(1, bucket + 1)) if trial % 3 else int(rng.integers(1, 8))
        x = gradient_like(n, seed=trial, ties=bool(trial % 2))
        ef_h = synth.host_normal(n, 1e-4, seed=trial + 1000)
        ef_d = dev_ef(ef_h)
        vals, idx = run_topk(qc, x, ef_d, bucket, k)
        pv, pi = ora.encode_topk(x, ef_h, bucket, k)
        assert bits_equal(idx.host().view(np.uint32), pi), (trial, n, bucket, k)
        assert bits_equal(vals.f32(), pv), (trial, n, bucket, k)
        assert bits_equal(ef_d.f32(), ef_h), (trial, n, bucket, k)


def sparse_workers(m, n, bucket, k, rng, mode):
    """m workers' pairs for the sum.  mode "random": independent gradients;
    "same": every worker sends the same indices (each index is hit m
    times); "alias": indices that agree modulo 1024; "mixed": some
    workers share indices, some do not, some slots are unused."""
    nb = -(-n // bucket)
    V = np.zeros((m, nb * k), np.float32)
    I = np.full((m, nb * k), 0xFFFFFFFF, np.uint32)
    for b in range(nb):
        cnt = min(bucket, n - b * bucket)
        kb = min(k, cnt)
        common = rng.choice(cnt, kb, replace=False)
        for w in range(m):
            if mode == "same":
                pick = common
            elif mode == "alias":
                base = rng.integers(0, min(cnt, 1024))
                pick = np.unique((base + 1024 * np.arange(kb)) % cnt)[:kb]
            elif mode == "mixed" and w % 3:
                pick = common if w % 2 else rng.choice(cnt, kb, replace=False)
                pick = pick[: kb - (w % 2)] if kb > 1 else pick
            else:
                pick = rng.choice(cnt, kb, replace=False)
            pick = np.sort(pick)
            vals = synth.host_normal(pick.size, 1.0, seed=int(rng.integers(1 << 30)))
            vals[::5] = -0.0
            V[w, b * k: b * k + pick.size] = vals
            I[w, b * k: b * k + pick.size] = pick
    return V.reshape(-1), I.reshape(-1)


@pytest.mark.parametrize("mode", ["random", "same", "alias", "mixed"])
@pytest.mark.parametrize("bucket,k,m,nbk", [(64, 1, 600, 3), (256, 63, 9, 9), (1024, 10, 100, 17),
                                            (4096, 4, 64, 5), (8192, 33, 20, 2), (2048, 1, 3, 1),
                                            (32768, 5, 40, 2)])
def test_topk_sum_conflicts(qc, ora, mode, bucket, k, m, nbk):
    """The one-wave sum for k < 64: several chunks of 256 pairs per bucket,
    one worker per pair (k = 1, 600 workers), every worker on the same
    indices, indices equal modulo the tag table's size, fewer buckets than
    XCDs, a short last bucket, and a continued sum."""
    rng = np.random.default_rng(bucket + k + m + len(mode))
    n = nbk * bucket - (bucket // 3 if nbk > 1 else 0)
    V, I = sparse_workers(m, n, bucket, k, rng, mode)
    acc = out_f32(n)
    qc.qc_topk_accumulate(dev(V), dev(I.view(np.int32)), m, n, bucket, k, acc.t, False)
    sync()
    want = ora.topk_accumulate(V, I, m, n, bucket, k)
    assert bits_equal(acc.f32(), want), first_diff(acc.f32(), want)
    start = synth.host_normal(n, 1.0, seed=m)
    start[::7] = -0.0
    acc.t.copy_(dev(start))
    qc.qc_topk_accumulate(dev(V), dev(I.view(np.int32)), m, n, bucket, k, acc.t, True)
    sync()
    want2 = ora.topk_accumulate(V, I, m, n, bucket, k, acc=start)
    assert bits_equal(acc.f32(), want2), first_diff(acc.f32(), want2)
