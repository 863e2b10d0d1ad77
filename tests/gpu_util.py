"""Device-buffer helpers for the GPU tests: outputs are pre-filled with a
sentinel (so an unwritten byte shows up) and followed by a canary band (so
a write past the end shows up)."""
import numpy as np
import pytest

SENTINEL = 0xA5
CANARY = 0x5C
GUARD = 256  # bytes of canary after every output buffer


def need_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import embedding_communication_codecs_amd as qc

    qc.lib()  # raises if the HIP library is missing: no fallback
    return qc


class Out:
    """An output buffer of `nbytes` (viewed as `dtype`) with a canary band."""

    def __init__(self, nbytes, dtype=None):
        import torch

        self.nbytes = nbytes
        self.raw = torch.full((nbytes + GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
        self.raw[nbytes:] = CANARY
        self.dtype = dtype or torch.uint8

    @property
    def t(self):
        return self.raw[: self.nbytes].view(self.dtype)

    def host(self):
        """Bytes of the buffer (checks the canary band is intact)."""
        h = self.raw.cpu().numpy()
        assert np.all(h[self.nbytes:] == CANARY), "write past the end of an output buffer"
        return h[: self.nbytes].copy()

    def f32(self):
        return self.host().view(np.float32)


def out_f32(count):
    import torch

    return Out(4 * count, torch.float32)


def dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_ef(a):
    """A device copy of an fp32 residual buffer (followed by a canary band)."""
    import torch

    o = out_f32(a.size)
    o.t.copy_(torch.from_numpy(np.ascontiguousarray(a, np.float32)))
    return o


def bits_equal(a, b):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


def first_diff(a, b):
    av = np.ascontiguousarray(a).view(np.uint32 if a.dtype == np.float32 else np.uint8)
    bv = np.ascontiguousarray(b).view(np.uint32 if b.dtype == np.float32 else np.uint8)
    idx = np.nonzero(av != bv)[0]
    if idx.size == 0:
        return "identical"
    i = idx[0]
    return f"{idx.size} differences, first at {i}: gpu={a[i]!r} oracle={b[i]!r}"
