"""ctypes binding of libqc with the C ABI's names (see include/qc.h).

Argument marshalling only: every codec step runs in the HIP kernels behind
the C ABI.  Array arguments may be torch tensors (their device pointer is
passed) or plain integers (raw device addresses, passed unchecked).  For
tensors the binding also checks that each buffer is on the GPU, contiguous
and large enough for what the call will read or write, so a size mistake is
a Python exception instead of an out-of-bounds access.  A non-zero status
from the library raises QcError.  There is no CPU fallback: if libqc.so has
not been built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqc.so")

QC_OK, QC_ERR_ARG, QC_ERR_ALIGN, QC_ERR_UNSUPPORTED, QC_ERR_LAUNCH = 0, 1, 2, 3, 4
QC_UNIFORM, QC_FP8_ROWWISE, QC_QSGD, QC_SIGN, QC_TERNARY, QC_INT8_SHARED = 0, 1, 2, 3, 4, 5
QC_F32, QC_BF16 = 0, 1
QC_MIN_BUCKET, QC_MAX_BUCKET, QC_MAX_WORKERS = 64, 65536, 65535
QC_INDEX_SHIFT = 12
QC_MAX_LIST_BUCKET = 32768
QC_MAX_TOPK_BUCKET = 65536

EXPORTS = (
    "qc_encode_uniform", "qc_encode_uniform_stochastic", "qc_encode_uniform_multi", "qc_encode_fp8_rowwise",
    "qc_encode_qsgd",
    "qc_encode_ternary", "qc_encode_sign", "qc_bucket_absmax", "qc_absmax_combine", "qc_encode_int8_shared",
    "qc_sum_int8_shared", "qc_tensor_index", "qc_encode_topk", "qc_decode_topk", "qc_topk_accumulate",
    "qc_encode_uniform_stochastic_multi", "qc_encode_qsgd_multi", "qc_encode_ternary_multi", "qc_encode_sign_multi",
    "qc_bucket_absmax_multi", "qc_encode_int8_shared_multi", "qc_encode_topk_multi",
    "qc_decode", "qc_decode_multi", "qc_dequant_accumulate", "qc_majority_vote", "qc_payload_bytes", "qc_status_str",
)


class QcError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libqc.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m embedding_communication_codecs_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, U64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
        sig = {
            "qc_encode_uniform": [P, P, I64, I32, I32, P, P, P, P],
            "qc_encode_uniform_stochastic": [P, P, I64, I32, I32, U64, U64, P, P, P, P],
            "qc_encode_ternary": [P, P, I64, I32, U64, U64, P, P, P],
            "qc_tensor_index": [P, I32, P, P],
            "qc_encode_topk": [P, P, I64, I32, I32, P, P, P],
            "qc_decode_topk": [P, P, I64, I32, I32, P, P],
            "qc_topk_accumulate": [P, P, I32, I64, I32, I32, P, I32, P],
            "qc_encode_uniform_multi": [P, P, P, I32, I64, P, I32, I32, P, P, P, P],
            "qc_encode_uniform_stochastic_multi": [P, P, P, I32, I64, P, I32, I32, U64, U64, P, P, P, P],
            "qc_encode_qsgd_multi": [P, P, P, I32, I64, P, I32, I32, U64, U64, P, P, P],
            "qc_encode_ternary_multi": [P, P, P, I32, I64, P, I32, U64, U64, P, P, P],
            "qc_encode_sign_multi": [P, I32, P, P, I32, I64, P, I32, P, P, P],
            "qc_bucket_absmax_multi": [P, P, P, I32, I64, P, I32, P, P],
            "qc_encode_int8_shared_multi": [P, P, P, I32, I64, P, I32, P, P, P, P],
            "qc_encode_topk_multi": [P, P, P, I32, I64, P, I32, I32, P, P, P],
            "qc_decode_multi": [I32, P, P, P, I64, I32, I32, P, P, P, I32, P],
            "qc_encode_fp8_rowwise": [P, I64, I32, P, P, P],
            "qc_encode_qsgd": [P, P, I64, I32, I32, U64, U64, P, P, P],
            "qc_encode_sign": [P, I32, P, I64, I32, P, P, P],
            "qc_decode": [I32, P, P, P, I64, I32, I32, P, P],
            "qc_dequant_accumulate": [I32, P, P, P, I32, I64, I32, I32, P, I32, P, P, P, P],
            "qc_majority_vote": [P, I32, I64, P, P],
            "qc_bucket_absmax": [P, P, I64, I32, P, P],
            "qc_absmax_combine": [P, I32, I64, P, P],
            "qc_encode_int8_shared": [P, P, I64, I32, P, P, P, P],
            "qc_sum_int8_shared": [P, I32, I64, I32, P, P, I32, P, P],
            "qc_payload_bytes": [I32, I64, I32, I32],
            "qc_status_str": [I32],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.qc_payload_bytes.restype = I64
        L.qc_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


# ----------------------------------------------------------------- helpers


def payload_bytes(fmt: int, n: int, group: int = 64, bits: int = 8) -> int:
    return int(lib().qc_payload_bytes(fmt, n, group, bits))


def nbuckets(n: int, group: int) -> int:
    return -(-n // group)


def _bytes(t) -> int:
    return t.numel() * t.element_size()


def _ptr(t, need_bytes: int | None, name: str):
    """Device address of a tensor/int/None, checking capacity for tensors."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if need_bytes is not None and _bytes(t) < need_bytes:
        raise ValueError(f"{name} holds {_bytes(t)} bytes, the call needs {need_bytes}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != QC_OK:
        raise QcError(status, lib().qc_status_str(status).decode())


# ------------------------------------------------------------ entry points


UNIFORM_BITS = (2, 4, 8)


def qc_encode_uniform(x, ef, n, bucket, bits, codes, scale, zero, stream=None):
    nb = nbuckets(n, bucket) if n > 0 and bucket > 0 else 0
    pb = payload_bytes(QC_UNIFORM, n, bucket, bits) if bits in UNIFORM_BITS and n >= 0 else None
    _check(lib().qc_encode_uniform(
        _ptr(x, 4 * n, "x"), _ptr(ef, 4 * n, "ef"), n, bucket, bits, _ptr(codes, pb, "codes"),
        _ptr(scale, 4 * nb, "scale"), _ptr(zero, 4 * nb, "zero"), _stream(stream)))


def qc_encode_uniform_stochastic(x, ef, n, bucket, bits, seed, elem_offset, codes, scale, zero,
                                 stream=None):
    nb = nbuckets(n, bucket) if n > 0 and bucket > 0 else 0
    pb = payload_bytes(QC_UNIFORM, n, bucket, bits) if bits in UNIFORM_BITS and n >= 0 else None
    _check(lib().qc_encode_uniform_stochastic(
        _ptr(x, 4 * n, "x"), _ptr(ef, 4 * n, "ef"), n, bucket, bits, seed & (2**64 - 1), elem_offset,
        _ptr(codes, pb, "codes"), _ptr(scale, 4 * nb, "scale"), _ptr(zero, 4 * nb, "zero"),
        _stream(stream)))


def qc_encode_ternary(x, ef, n, bucket, seed, elem_offset, words, scale, stream=None):
    nb = nbuckets(n, bucket) if n > 0 and bucket > 0 else 0
    pb = payload_bytes(QC_TERNARY, n, bucket, 2) if n >= 0 else None
    _check(lib().qc_encode_ternary(
        _ptr(x, 4 * n, "x"), _ptr(ef, 4 * n, "ef"), n, bucket, seed & (2**64 - 1), elem_offset,
        _ptr(words, pb, "words"), _ptr(scale, 4 * nb, "scale"), _stream(stream)))


class TensorTable:
    """Device tables describing a list of GPU tensors of one dtype (float32,
    or bfloat16 for the sign encoder) as one buffer: `xs` (int64 data
    pointers), and the bucket plan qc_tensor_index builds on the host,
    `offsets` (prefix sums of the sizes, length ntensors + 1) and
    `seg_first`.  Build it once per list layout and reuse it; it keeps the
    tensors alive."""

    def __init__(self, tensors):
        import torch

        if not tensors:
            raise ValueError("empty tensor list")
        self.dtype = tensors[0].dtype
        if self.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("tensors must be float32 or bfloat16")
        sizes = []
        for k, t in enumerate(tensors):
            if not t.is_cuda or t.dtype != self.dtype or not t.is_contiguous():
                raise ValueError(f"tensor {k} must be a contiguous {self.dtype} GPU tensor like tensor 0")
            if t.data_ptr() % t.element_size():
                raise ValueError(f"tensor {k} is not aligned to its element size")
            sizes.append(t.numel())
        import numpy as np

        self.tensors = list(tensors)
        self.ntensors = len(sizes)
        self.n = int(sum(sizes))
        host_sizes = np.array(sizes, dtype=np.int64)
        offs = np.empty(self.ntensors + 1, dtype=np.int64)
        nseg = -(-self.n // (1 << QC_INDEX_SHIFT))
        seg = np.empty(nseg + 1, dtype=np.int32)
        _check(lib().qc_tensor_index(host_sizes.ctypes.data, self.ntensors, offs.ctypes.data, seg.ctypes.data))
        dev = tensors[0].device
        self.xs = torch.tensor([t.data_ptr() for t in tensors], dtype=torch.int64, device=dev)
        self.offsets = torch.from_numpy(offs).to(dev)
        self.seg_first = torch.from_numpy(seg).to(dev)


def _nseg(n):
    return -(-max(n, 0) // (1 << QC_INDEX_SHIFT)) + 1


def qc_tensor_index(sizes, ntensors, offsets, seg_first) -> None:
    """Host arrays (numpy): sizes int64[ntensors] in, offsets int64[ntensors+1]
    and seg_first int32[nseg+1] out."""
    _check(lib().qc_tensor_index(sizes.ctypes.data, ntensors, offsets.ctypes.data, seg_first.ctypes.data))


def qc_encode_uniform_multi(xs, offsets, seg_first, ntensors, n, ef, bucket, bits, codes, scale, zero,
                            stream=None):
    """xs/offsets/seg_first: device tables (see TensorTable) or raw addresses."""
    nb = nbuckets(n, bucket) if n > 0 and bucket > 0 else 0
    pb = payload_bytes(QC_UNIFORM, n, bucket, bits) if bits in UNIFORM_BITS and n >= 0 else None
    _check(lib().qc_encode_uniform_multi(
        _ptr(xs, 8 * max(ntensors, 0), "xs"), _ptr(offsets, 8 * (max(ntensors, 0) + 1), "offsets"),
        _ptr(seg_first, 4 * _nseg(n), "seg_first"), ntensors, n, _ptr(ef, 4 * n, "ef"), bucket, bits,
        _ptr(codes, pb, "codes"), _ptr(scale, 4 * nb, "scale"), _ptr(zero, 4 * nb, "zero"), _stream(stream)))


def _list_args(xs, offsets, seg_first, ntensors, n):
    return (_ptr(xs, 8 * max(ntensors, 0), "xs"), _ptr(offsets, 8 * (max(ntensors, 0) + 1), "offsets"),
            _ptr(seg_first, 4 * _nseg(n), "seg_first"), ntensors, n)


def qc_encode_uniform_stochastic_multi(xs, offsets, seg_first, ntensors, n, ef, bucket, bits, seed, elem_offset,
                                       codes, scale, zero, stream=None):
    nb = nbuckets(n, bucket) if n > 0 and bucket > 0 else 0
    pb = payload_bytes(QC_UNIFORM, n, bucket, bits) if bits in UNIFORM_BITS and n >= 0 else None
    _check(lib().qc_encode_uniform_stochastic_multi(
        *_list_args(xs, offsets, seg_first, ntensors, n), _ptr(ef, 4 * n, "ef"), bucket, bits,
        seed & (2**64 - 1), elem_offset, _ptr(codes, pb, "codes"), _ptr(scale, 4 * nb, "scale"),
        _ptr(zero, 4 * nb, "zero"), _stream(stream)))


def qc_encode_qsgd_multi(xs, offsets, seg_first, ntensors, n, ef, bucket, levels, seed, elem_offset, words, norm,
                         stream=None):
    nb = nbuckets(n, bucket) if n > 0 and bucket > 0 else 0
    pb = payload_bytes(QC_QSGD, n, bucket, 16) if n >= 0 else None
    _check(lib().qc_encode_qsgd_multi(
        *_list_args(xs, offsets, seg_first, ntensors, n), _ptr(ef, 4 * n, "ef"), bucket, levels,
        seed & (2**64 - 1), elem_offset, _ptr(words, pb, "words"), _ptr(norm, 4 * nb, "norm"), _stream(stream)))


def qc_encode_ternary_multi(xs, offsets, seg_first, ntensors, n, ef, bucket, seed, elem_offset, words, scale,
                            stream=None):
    nb = nbuckets(n, bucket) if n > 0 and bucket > 0 else 0
    pb = payload_bytes(QC_TERNARY, n, bucket, 2) if n >= 0 else None
    _check(lib().qc_encode_ternary_multi(
        *_list_args(xs, offsets, seg_first, ntensors, n), _ptr(ef, 4 * n, "ef"), bucket, seed & (2**64 - 1),
        elem_offset, _ptr(words, pb, "words"), _ptr(scale, 4 * nb, "scale"), _stream(stream)))


def qc_encode_sign_multi(xs, xtype, offsets, seg_first, ntensors, n, ef, bucket, words, scale, stream=None):
    nb = nbuckets(n, bucket) if n > 0 and bucket > 0 else 0
    pb = payload_bytes(QC_SIGN, n, bucket, 1) if n >= 0 else None
    a = _list_args(xs, offsets, seg_first, ntensors, n)
    _check(lib().qc_encode_sign_multi(
        a[0], xtype, *a[1:], _ptr(ef, 4 * n, "ef"), bucket, _ptr(words, pb, "words"), _ptr(scale, 4 * nb, "scale"),
        _stream(stream)))


def qc_bucket_absmax_multi(xs, offsets, seg_first, ntensors, n, ef, bucket, amax, stream=None):
    nb = nbuckets(n, bucket) if n > 0 and bucket > 0 else 0
    _check(lib().qc_bucket_absmax_multi(
        *_list_args(xs, offsets, seg_first, ntensors, n), _ptr(ef, 4 * n, "ef"), bucket, _ptr(amax, 4 * nb, "amax"),
        _stream(stream)))


def qc_encode_int8_shared_multi(xs, offsets, seg_first, ntensors, n, ef, bucket, amax, codes, scale, stream=None):
    nb = nbuckets(n, bucket) if n > 0 and bucket > 0 else 0
    pb = payload_bytes(QC_INT8_SHARED, n, bucket, 8) if n >= 0 else None
    _check(lib().qc_encode_int8_shared_multi(
        *_list_args(xs, offsets, seg_first, ntensors, n), _ptr(ef, 4 * n, "ef"), bucket, _ptr(amax, 4 * nb, "amax"),
        _ptr(codes, pb, "codes"), _ptr(scale, 4 * nb, "scale"), _stream(stream)))


def qc_encode_fp8_rowwise(x, rows, dim, codes, scale, stream=None):
    n = rows * dim
    pb = payload_bytes(QC_FP8_ROWWISE, n, dim, 8) if n >= 0 else None
    _check(lib().qc_encode_fp8_rowwise(
        _ptr(x, 4 * n, "x"), rows, dim, _ptr(codes, pb, "codes"), _ptr(scale, 4 * max(rows, 0), "scale"),
        _stream(stream)))


def qc_encode_qsgd(x, ef, n, bucket, levels, seed, elem_offset, words, norm, stream=None):
    nb = nbuckets(n, bucket) if n > 0 and bucket > 0 else 0
    pb = payload_bytes(QC_QSGD, n, bucket, 16) if n >= 0 else None
    _check(lib().qc_encode_qsgd(
        _ptr(x, 4 * n, "x"), _ptr(ef, 4 * n, "ef"), n, bucket, levels, seed & (2**64 - 1),
        elem_offset, _ptr(words, pb, "words"), _ptr(norm, 4 * nb, "norm"), _stream(stream)))


def qc_encode_sign(x, xtype, ef, n, bucket, words, scale, stream=None):
    nb = nbuckets(n, bucket) if n > 0 and bucket > 0 else 0
    pb = payload_bytes(QC_SIGN, n, bucket, 1) if n >= 0 else None
    xbytes = (2 if xtype == QC_BF16 else 4) * n
    _check(lib().qc_encode_sign(
        _ptr(x, xbytes, "x"), xtype, _ptr(ef, 4 * n, "ef"), n, bucket, _ptr(words, pb, "words"),
        _ptr(scale, 4 * nb, "scale"), _stream(stream)))


def qc_decode(fmt, codes, scale, zero, n, group, bits, out, stream=None):
    nb = nbuckets(n, group) if n > 0 and group > 0 else 0
    pb = payload_bytes(fmt, n, group, bits) if n >= 0 else -1
    _check(lib().qc_decode(
        fmt, _ptr(codes, pb if pb >= 0 else None, "codes"), _ptr(scale, 4 * nb, "scale"),
        _ptr(zero, 4 * nb, "zero"), n, group, bits, _ptr(out, 4 * n, "out"), _stream(stream)))


def qc_decode_multi(fmt, codes, scale, zero, n, group, bits, outs, offsets, seg_first, ntensors, stream=None):
    """outs/offsets/seg_first: device tables (see TensorTable) or raw addresses."""
    nb = nbuckets(n, group) if n > 0 and group > 0 else 0
    pb = payload_bytes(fmt, n, group, bits) if n >= 0 else -1
    _check(lib().qc_decode_multi(
        fmt, _ptr(codes, pb if pb >= 0 else None, "codes"), _ptr(scale, 4 * nb, "scale"),
        _ptr(zero, 4 * nb, "zero"), n, group, bits, _ptr(outs, 8 * max(ntensors, 0), "outs"),
        _ptr(offsets, 8 * (max(ntensors, 0) + 1), "offsets"), _ptr(seg_first, 4 * _nseg(n), "seg_first"),
        ntensors, _stream(stream)))


def qc_dequant_accumulate(fmt, codes, scale, zero, m, n, group, bits, acc, accumulate,
                          rq_codes=None, rq_scale=None, rq_zero=None, stream=None):
    nb = nbuckets(n, group) if n > 0 and group > 0 else 0
    pb = payload_bytes(fmt, n, group, bits) if n >= 0 else -1
    mm = max(m, 0)
    rq_pb = payload_bytes(QC_UNIFORM, n, group, bits) if bits in UNIFORM_BITS and n >= 0 else None
    _check(lib().qc_dequant_accumulate(
        fmt, _ptr(codes, mm * pb if pb >= 0 else None, "codes"), _ptr(scale, 4 * mm * nb, "scale"),
        _ptr(zero, 4 * mm * nb, "zero"), m, n, group, bits, _ptr(acc, 4 * n, "acc"),
        1 if accumulate else 0, _ptr(rq_codes, rq_pb, "rq_codes"), _ptr(rq_scale, 4 * nb, "rq_scale"),
        _ptr(rq_zero, 4 * nb, "rq_zero"), _stream(stream)))


def qc_bucket_absmax(x, ef, n, bucket, amax, stream=None):
    nb = nbuckets(n, bucket) if n > 0 and bucket > 0 else 0
    _check(lib().qc_bucket_absmax(_ptr(x, 4 * n, "x"), _ptr(ef, 4 * n, "ef"), n, bucket,
                                  _ptr(amax, 4 * nb, "amax"), _stream(stream)))


def qc_absmax_combine(amax, m, nb, out, stream=None):
    _check(lib().qc_absmax_combine(_ptr(amax, 4 * max(m, 0) * max(nb, 0), "amax"), m, nb,
                                   _ptr(out, 4 * max(nb, 0), "out"), _stream(stream)))


def qc_encode_int8_shared(x, ef, n, bucket, amax, codes, scale, stream=None):
    nb = nbuckets(n, bucket) if n > 0 and bucket > 0 else 0
    pb = payload_bytes(QC_INT8_SHARED, n, bucket, 8) if n >= 0 else None
    _check(lib().qc_encode_int8_shared(
        _ptr(x, 4 * n, "x"), _ptr(ef, 4 * n, "ef"), n, bucket, _ptr(amax, 4 * nb, "amax"),
        _ptr(codes, pb, "codes"), _ptr(scale, 4 * nb, "scale"), _stream(stream)))


def qc_sum_int8_shared(codes, m, n, bucket, scale, isum, accumulate, out, stream=None):
    nb = nbuckets(n, bucket) if n > 0 and bucket > 0 else 0
    pb = payload_bytes(QC_INT8_SHARED, n, bucket, 8) if n >= 0 else None
    _check(lib().qc_sum_int8_shared(
        _ptr(codes, max(m, 0) * pb if pb is not None else None, "codes"), m, n, bucket,
        _ptr(scale, 4 * nb, "scale"), _ptr(isum, 4 * max(n, 0), "isum"), 1 if accumulate else 0,
        _ptr(out, 4 * max(n, 0), "out"), _stream(stream)))


def qc_encode_topk(x, ef, n, bucket, k, values, indices, stream=None):
    slots = nbuckets(n, bucket) * k if n > 0 and bucket > 0 and k > 0 else 0
    _check(lib().qc_encode_topk(_ptr(x, 4 * n, "x"), _ptr(ef, 4 * n, "ef"), n, bucket, k,
                                _ptr(values, 4 * slots, "values"), _ptr(indices, 4 * slots, "indices"),
                                _stream(stream)))


def qc_encode_topk_multi(xs, offsets, seg_first, ntensors, n, ef, bucket, k, values, indices, stream=None):
    slots = nbuckets(n, bucket) * k if n > 0 and bucket > 0 and k > 0 else 0
    _check(lib().qc_encode_topk_multi(
        *_list_args(xs, offsets, seg_first, ntensors, n), _ptr(ef, 4 * n, "ef"), bucket, k,
        _ptr(values, 4 * slots, "values"), _ptr(indices, 4 * slots, "indices"), _stream(stream)))


def qc_decode_topk(values, indices, n, bucket, k, out, stream=None):
    slots = nbuckets(n, bucket) * k if n > 0 and bucket > 0 and k > 0 else 0
    _check(lib().qc_decode_topk(_ptr(values, 4 * slots, "values"), _ptr(indices, 4 * slots, "indices"), n,
                                bucket, k, _ptr(out, 4 * max(n, 0), "out"), _stream(stream)))


def qc_topk_accumulate(values, indices, m, n, bucket, k, acc, accumulate, stream=None):
    slots = max(m, 0) * (nbuckets(n, bucket) * k if n > 0 and bucket > 0 and k > 0 else 0)
    _check(lib().qc_topk_accumulate(_ptr(values, 4 * slots, "values"), _ptr(indices, 4 * slots, "indices"), m,
                                    n, bucket, k, _ptr(acc, 4 * max(n, 0), "acc"), 1 if accumulate else 0,
                                    _stream(stream)))


def qc_majority_vote(words, m, n, out_words, stream=None):
    pb = payload_bytes(QC_SIGN, n, 64, 1) if n >= 0 else None
    _check(lib().qc_majority_vote(
        _ptr(words, max(m, 0) * pb if pb is not None else None, "words"), m, n,
        _ptr(out_words, pb, "out_words"), _stream(stream)))


def qc_payload_bytes(fmt, n, group, bits) -> int:
    return int(lib().qc_payload_bytes(fmt, n, group, bits))


def qc_status_str(status) -> str:
    return lib().qc_status_str(status).decode()
