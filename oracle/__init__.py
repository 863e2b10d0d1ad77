"""CPU oracle for the quantized-communication codec (ctypes over numpy).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  The GPU library neither imports nor links it, and the two share
no source.

The arithmetic lives in ``qc_oracle.c`` (plain single-threaded C, fp32,
no FMA contraction); this module only builds it with gcc and marshals numpy
arrays.  Every function returns fresh numpy arrays; ``ef`` arrays are updated
in place, exactly as the C functions do.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qc_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

UNIFORM, FP8_ROWWISE, QSGD, SIGN, TERNARY, INT8_SHARED = 0, 1, 2, 3, 4, 5

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (always when ``force``)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        stale = os.path.exists(LIB) and any(
            os.path.getmtime(s) > os.path.getmtime(LIB)
            for s in (SRC, os.path.join(HERE, "qc_oracle.h")))
        if stale or not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        P, I64, I32, U64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64
        L.qco_payload_bytes.argtypes = [I32, I64, I32]
        L.qco_payload_bytes.restype = I64
        L.qco_philox4x32_10.argtypes = [P, P, P]
        L.qco_e4m3_from_f32.argtypes = [ctypes.c_float]
        L.qco_e4m3_from_f32.restype = ctypes.c_uint8
        L.qco_e4m3_from_f32_n.argtypes = [P, I64, P]
        L.qco_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        L.qco_e4m3_to_f32.restype = ctypes.c_float
        L.qco_tree_sum.argtypes = [P, I64, I64]
        L.qco_tree_sum.restype = ctypes.c_float
        L.qco_encode_uniform.argtypes = [P, P, I64, I32, I32, P, P, P]
        L.qco_decode_uniform.argtypes = [P, P, P, I64, I32, I32, P]
        L.qco_encode_uniform_stochastic.argtypes = [P, P, I64, I32, I32, U64, U64, P, P, P]
        L.qco_encode_ternary.argtypes = [P, P, I64, I32, U64, U64, P, P]
        L.qco_decode_ternary.argtypes = [P, P, I64, I32, P]
        L.qco_encode_fp8_rowwise.argtypes = [P, I64, I32, P, P]
        L.qco_decode_fp8_rowwise.argtypes = [P, P, I64, I32, P]
        L.qco_encode_qsgd.argtypes = [P, P, I64, I32, U64, U64, P, P]
        L.qco_decode_qsgd.argtypes = [P, P, I64, I32, P]
        L.qco_encode_sign.argtypes = [P, I32, P, I64, I32, P, P]
        L.qco_decode_sign.argtypes = [P, P, I64, I32, P]
        L.qco_decode_one.argtypes = [I32, P, P, P, I64, I32, I32]
        L.qco_decode_one.restype = ctypes.c_float
        L.qco_dequant_accumulate.argtypes = [I32, P, P, P, I32, I64, I32, I32, P, I32]
        L.qco_majority_vote.argtypes = [P, I32, I64, P]
        L.qco_bucket_absmax.argtypes = [P, P, I64, I32, P]
        L.qco_absmax_combine.argtypes = [P, I32, I64, P]
        L.qco_encode_int8_shared.argtypes = [P, P, I64, I32, P, P, P]
        L.qco_decode_int8_shared.argtypes = [P, P, I64, I32, P]
        L.qco_sum_int8_shared.argtypes = [P, I32, I64, I32, P, P, I32, P]
        L.qco_encode_topk.argtypes = [P, P, I64, I32, I32, P, P]
        L.qco_decode_topk.argtypes = [P, P, I64, I32, I32, P]
        L.qco_topk_accumulate.argtypes = [P, P, I32, I64, I32, I32, P, I32]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _ef(ef):
    if ef is None:
        return None
    if ef.dtype != np.float32 or not ef.flags.c_contiguous:
        raise TypeError("ef must be a contiguous float32 array (updated in place)")
    return ef


def nbuckets(n: int, group: int) -> int:
    return -(-n // group)


def payload_bytes(fmt: int, n: int, bits: int = 8) -> int:
    return int(lib().qco_payload_bytes(fmt, n, bits))


def philox4x32_10(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().qco_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def e4m3_from_f32(y: float) -> int:
    return int(lib().qco_e4m3_from_f32(ctypes.c_float(y)))


def e4m3_from_f32_n(y) -> np.ndarray:
    """Codes of an array (each value clamped to [-448, 448] first)."""
    y = _f32(y)
    out = np.empty(y.size, dtype=np.uint8)
    lib().qco_e4m3_from_f32_n(_p(y), y.size, _p(out))
    return out


def e4m3_to_f32(c: int) -> float:
    return float(np.float32(lib().qco_e4m3_to_f32(c)))


def tree_sum(terms, pow2len: int) -> np.float32:
    t = _f32(terms)
    return np.float32(lib().qco_tree_sum(_p(t), t.size, pow2len))


def encode_uniform(x, ef, bucket: int, bits: int):
    x = _f32(x)
    ef = _ef(ef)
    n = x.size
    nb = nbuckets(n, bucket)
    payload = np.empty(payload_bytes(UNIFORM, n, bits), dtype=np.uint8)
    scale = np.empty(nb, dtype=np.float32)
    zero = np.empty(nb, dtype=np.float32)
    lib().qco_encode_uniform(_p(x), _p(ef), n, bucket, bits, _p(payload), _p(scale), _p(zero))
    return payload, scale, zero


def encode_uniform_stochastic(x, ef, bucket: int, bits: int, seed: int, elem_offset: int = 0):
    x = _f32(x)
    ef = _ef(ef)
    n = x.size
    nb = nbuckets(n, bucket)
    payload = np.empty(payload_bytes(UNIFORM, n, bits), dtype=np.uint8)
    scale = np.empty(nb, dtype=np.float32)
    zero = np.empty(nb, dtype=np.float32)
    lib().qco_encode_uniform_stochastic(_p(x), _p(ef), n, bucket, bits, seed & (2**64 - 1), elem_offset,
                                        _p(payload), _p(scale), _p(zero))
    return payload, scale, zero


def encode_ternary(x, ef, bucket: int, seed: int, elem_offset: int = 0):
    x = _f32(x)
    ef = _ef(ef)
    n = x.size
    payload = np.empty(payload_bytes(TERNARY, n, 2), dtype=np.uint8)
    scale = np.empty(nbuckets(n, bucket), dtype=np.float32)
    lib().qco_encode_ternary(_p(x), _p(ef), n, bucket, seed & (2**64 - 1), elem_offset, _p(payload),
                             _p(scale))
    return payload, scale


def decode_ternary(payload, scale, n: int, bucket: int):
    out = np.empty(n, dtype=np.float32)
    lib().qco_decode_ternary(_p(np.ascontiguousarray(payload, np.uint8)), _p(_f32(scale)), n, bucket,
                             _p(out))
    return out


def decode_uniform(payload, scale, zero, n: int, bucket: int, bits: int):
    out = np.empty(n, dtype=np.float32)
    lib().qco_decode_uniform(_p(np.ascontiguousarray(payload, np.uint8)), _p(_f32(scale)),
                             _p(_f32(zero)), n, bucket, bits, _p(out))
    return out


def encode_fp8_rowwise(x, rows: int, dim: int):
    x = _f32(x)
    assert x.size == rows * dim
    payload = np.empty(payload_bytes(FP8_ROWWISE, rows * dim), dtype=np.uint8)
    scale = np.empty(rows, dtype=np.float32)
    lib().qco_encode_fp8_rowwise(_p(x), rows, dim, _p(payload), _p(scale))
    return payload, scale


def decode_fp8_rowwise(payload, scale, rows: int, dim: int):
    out = np.empty(rows * dim, dtype=np.float32)
    lib().qco_decode_fp8_rowwise(_p(np.ascontiguousarray(payload, np.uint8)), _p(_f32(scale)),
                                 rows, dim, _p(out))
    return out


def encode_qsgd(x, ef, bucket: int, seed: int, elem_offset: int = 0):
    x = _f32(x)
    ef = _ef(ef)
    n = x.size
    if elem_offset % 4:
        raise ValueError("elem_offset must be a multiple of 4")
    payload = np.empty(payload_bytes(QSGD, n, 4), dtype=np.uint8)
    norm = np.empty(nbuckets(n, bucket), dtype=np.float32)
    lib().qco_encode_qsgd(_p(x), _p(ef), n, bucket, seed & (2**64 - 1), elem_offset,
                          _p(payload), _p(norm))
    return payload, norm


def decode_qsgd(payload, norm, n: int, bucket: int):
    out = np.empty(n, dtype=np.float32)
    lib().qco_decode_qsgd(_p(np.ascontiguousarray(payload, np.uint8)), _p(_f32(norm)), n, bucket,
                          _p(out))
    return out


def encode_sign(x, ef, bucket: int):
    """x: float32 array, or uint16 array of bf16 bit patterns."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        is_bf16 = 1
    elif x.dtype == np.float32:
        is_bf16 = 0
    else:
        raise TypeError("x must be float32 or uint16 (bf16 bits)")
    ef = _ef(ef)
    n = x.size
    payload = np.empty(payload_bytes(SIGN, n, 1), dtype=np.uint8)
    scale = np.empty(nbuckets(n, bucket), dtype=np.float32)
    lib().qco_encode_sign(_p(x), is_bf16, _p(ef), n, bucket, _p(payload), _p(scale))
    return payload, scale


def decode_sign(payload, scale, n: int, bucket: int):
    out = np.empty(n, dtype=np.float32)
    lib().qco_decode_sign(_p(np.ascontiguousarray(payload, np.uint8)), _p(_f32(scale)), n, bucket,
                          _p(out))
    return out


def dequant_accumulate(fmt: int, payloads, scale, zero, m: int, n: int, group: int, bits: int,
                       acc=None):
    """payloads: uint8 [m * payload_bytes]; scale/zero: float32 [m * nb].
    If ``acc`` is given it is the starting value (accumulate=1) and is not
    modified; the result is returned as a new array."""
    payloads = np.ascontiguousarray(payloads, np.uint8)
    out = np.zeros(n, dtype=np.float32) if acc is None else _f32(acc).copy()
    z = None if zero is None else _f32(zero)
    lib().qco_dequant_accumulate(fmt, _p(payloads), _p(_f32(scale)), _p(z), m, n, group, bits,
                                 _p(out), 0 if acc is None else 1)
    return out


def majority_vote(payloads, m: int, n: int):
    payloads = np.ascontiguousarray(payloads, np.uint8)
    out = np.empty(payload_bytes(SIGN, n, 1), dtype=np.uint8)
    lib().qco_majority_vote(_p(payloads), m, n, _p(out))
    return out


# ------------------------------------------------------ shared-scale INT8


def bucket_absmax(x, ef, bucket: int):
    x = _f32(x)
    amax = np.empty(nbuckets(x.size, bucket), dtype=np.float32)
    lib().qco_bucket_absmax(_p(x), _p(None if ef is None else _f32(ef)), x.size, bucket, _p(amax))
    return amax


def absmax_combine(amax, m: int, nb: int):
    amax = _f32(amax)
    out = np.empty(nb, dtype=np.float32)
    lib().qco_absmax_combine(_p(amax), m, nb, _p(out))
    return out


def encode_int8_shared(x, ef, bucket: int, amax):
    """Returns (payload uint8, scale float32); ef (if given) is updated."""
    x = _f32(x)
    ef = _ef(ef)
    n = x.size
    payload = np.empty(payload_bytes(INT8_SHARED, n, 8), dtype=np.uint8)
    scale = np.empty(nbuckets(n, bucket), dtype=np.float32)
    lib().qco_encode_int8_shared(_p(x), _p(ef), n, bucket, _p(_f32(amax)), _p(payload), _p(scale))
    return payload, scale


def decode_int8_shared(payload, scale, n: int, bucket: int):
    out = np.empty(n, dtype=np.float32)
    lib().qco_decode_int8_shared(_p(np.ascontiguousarray(payload, np.uint8)), _p(_f32(scale)), n, bucket,
                                 _p(out))
    return out


def sum_int8_shared(payloads, m: int, n: int, bucket: int, scale, isum=None):
    """Returns (isum int32, out float32).  If ``isum`` is given it is the
    running integer sum to continue from (it is not modified)."""
    payloads = np.ascontiguousarray(payloads, np.uint8)
    acc = np.zeros(n, dtype=np.int32) if isum is None else np.array(isum, dtype=np.int32, copy=True)
    out = np.empty(n, dtype=np.float32)
    lib().qco_sum_int8_shared(_p(payloads), m, n, bucket, _p(_f32(scale)), _p(acc), 0 if isum is None else 1,
                              _p(out))
    return acc, out


# ----------------------------------------------------------------- top-k


def encode_topk(x, ef, bucket: int, k: int):
    """Returns (values float32[nb*k], indices uint32[nb*k]); ef is updated."""
    x = _f32(x)
    ef = _ef(ef)
    nb = nbuckets(x.size, bucket)
    values = np.empty(nb * k, dtype=np.float32)
    indices = np.empty(nb * k, dtype=np.uint32)
    lib().qco_encode_topk(_p(x), _p(ef), x.size, bucket, k, _p(values), _p(indices))
    return values, indices


def decode_topk(values, indices, n: int, bucket: int, k: int):
    out = np.empty(n, dtype=np.float32)
    lib().qco_decode_topk(_p(_f32(values)), _p(np.ascontiguousarray(indices, np.uint32)), n, bucket, k, _p(out))
    return out


def topk_accumulate(values, indices, m: int, n: int, bucket: int, k: int, acc=None):
    out = np.zeros(n, dtype=np.float32) if acc is None else _f32(acc).copy()
    lib().qco_topk_accumulate(_p(_f32(values)), _p(np.ascontiguousarray(indices, np.uint32)), m, n, bucket, k,
                              _p(out), 0 if acc is None else 1)
    return out


# -------------------------------------------------- bucketing front-end
# [GCQC, "When it breaks".]  The page's remedy for per-tensor overhead is
# to gather a model's many gradient tensors into one bucketed buffer before
# compressing.  Reading: the tensors are concatenated in list order into one
# buffer, which is then encoded (or decoded and split back) exactly as a
# single buffer is.


def concat(tensors):
    return np.concatenate([np.asarray(t, dtype=np.float32).ravel() for t in tensors])


def encode_uniform_multi(tensors, ef, bucket: int, bits: int):
    return encode_uniform(concat(tensors), ef, bucket, bits)


def decode_flat(fmt: int, payload, scale, zero, n: int, group: int, bits: int):
    """Any format's decoder on one payload of n elements."""
    if fmt == UNIFORM:
        return decode_uniform(payload, scale, zero, n, group, bits)
    if fmt == FP8_ROWWISE:
        return decode_fp8_rowwise(payload, scale, n // group, group)
    if fmt == QSGD:
        return decode_qsgd(payload, scale, n, group)
    if fmt == SIGN:
        return decode_sign(payload, scale, n, group)
    if fmt == TERNARY:
        return decode_ternary(payload, scale, n, group)
    if fmt == INT8_SHARED:
        return decode_int8_shared(payload, scale, n, group)
    raise ValueError(fmt)


def decode_multi(fmt: int, payload, scale, zero, sizes, group: int, bits: int):
    """The decoded concatenation split back into tensors of `sizes`."""
    flat = decode_flat(fmt, payload, scale, zero, int(sum(sizes)), group, bits)
    return np.split(flat, np.cumsum(sizes)[:-1])
