"""Host-side checks of the C ABI: the library loads, exports every entry
point include/qc.h declares, sizes payloads as documented, and rejects bad
arguments with the documented status before touching the HIP runtime (so
these run without a GPU)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qc.h")


@pytest.fixture(scope="module")
def qc():
    import embedding_communication_codecs_amd as q

    if not os.path.exists(q.binding.LIB_PATH):
        pytest.skip("libqc.so not built (python -m embedding_communication_codecs_amd.build)")
    q.lib()
    return q


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qc_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points(qc):
    names = declared_functions()
    assert set(names) == set(qc.EXPORTS), names


def test_library_exports_every_declared_symbol(qc):
    out = subprocess.run(["nm", "-D", "--defined-only", qc.binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(qc.lib(), name) is not None


def test_payload_bytes_matches_oracle(qc, ora):
    for n in (0, 1, 3, 4, 15, 16, 17, 31, 32, 33, 127, 128, 129, 1000, 65536, 10**9):
        assert qc.qc_payload_bytes(qc.QC_UNIFORM, n, 64, 8) == ora.payload_bytes(ora.UNIFORM, n, 8)
        assert qc.qc_payload_bytes(qc.QC_UNIFORM, n, 64, 4) == ora.payload_bytes(ora.UNIFORM, n, 4)
        assert qc.qc_payload_bytes(qc.QC_UNIFORM, n, 64, 2) == ora.payload_bytes(ora.UNIFORM, n, 2)
        assert qc.qc_payload_bytes(qc.QC_TERNARY, n, 64, 2) == ora.payload_bytes(ora.TERNARY, n, 2)
        assert qc.qc_payload_bytes(qc.QC_INT8_SHARED, n, 64, 8) == ora.payload_bytes(ora.INT8_SHARED, n, 8)
        assert qc.qc_payload_bytes(qc.QC_FP8_ROWWISE, n, 4, 8) == ora.payload_bytes(ora.FP8_ROWWISE, n)
        assert qc.qc_payload_bytes(qc.QC_QSGD, n, 512, 16) == ora.payload_bytes(ora.QSGD, n, 4)
        assert qc.qc_payload_bytes(qc.QC_SIGN, n, 4096, 1) == ora.payload_bytes(ora.SIGN, n, 1)
    assert qc.qc_payload_bytes(qc.QC_UNIFORM, 10, 64, 3) == -1
    assert qc.qc_payload_bytes(9, 10, 64, 8) == -1
    assert qc.qc_payload_bytes(qc.QC_UNIFORM, -1, 64, 8) == -1


def test_status_strings(qc):
    for s in range(5):
        assert qc.qc_status_str(s).startswith("QC_")
    assert "unknown" in qc.qc_status_str(99)


# Fake device addresses: validation rejects the call before any use.
A = 1 << 20           # 16-byte aligned
MIS = (1 << 20) + 4   # misaligned
NULL = None


def call(qc, name, *args):
    return getattr(qc.lib(), name)(*args)


def test_encode_uniform_errors(qc):
    f = "qc_encode_uniform"
    ok = (A, A, 1000, 256, 8, A, A, A, None)
    assert call(qc, f, NULL, *ok[1:]) == qc.QC_ERR_ARG
    assert call(qc, f, A, A, -1, 256, 8, A, A, A, None) == qc.QC_ERR_ARG
    for bad in (0, 32, 100, 96, 131072, -64):
        assert call(qc, f, A, A, 1000, bad, 8, A, A, A, None) == qc.QC_ERR_ARG, bad
    for bits in (0, 1, 3, 5, 16):
        assert call(qc, f, A, A, 1000, 256, bits, A, A, A, None) == qc.QC_ERR_UNSUPPORTED
    assert call(qc, f, A, A, 1000, 256, 8, NULL, A, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, A, 1000, 256, 8, A, NULL, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, A, 1000, 256, 8, A, A, NULL, None) == qc.QC_ERR_ARG
    for pos in (0, 1, 5, 6, 7):
        args = list(ok)
        args[pos] = MIS
        assert call(qc, f, *args) == qc.QC_ERR_ALIGN, pos
    # empty input is a valid no-op, even with NULL buffers
    assert call(qc, f, NULL, NULL, 0, 256, 8, NULL, NULL, NULL, None) == qc.QC_OK


def test_encode_uniform_stochastic_errors(qc):
    f = "qc_encode_uniform_stochastic"
    ok = (A, A, 1000, 256, 2, 7, 8, A, A, A, None)
    assert call(qc, f, *ok[:6], 6, *ok[7:]) == qc.QC_ERR_ARG  # offset % 4
    assert call(qc, f, NULL, *ok[1:]) == qc.QC_ERR_ARG
    assert call(qc, f, A, A, 1000, 192, 2, 7, 8, A, A, A, None) == qc.QC_ERR_ARG
    for bits in (0, 1, 3, 16):
        assert call(qc, f, A, A, 1000, 256, bits, 7, 8, A, A, A, None) == qc.QC_ERR_UNSUPPORTED
    for pos in (7, 8, 9):
        args = list(ok)
        args[pos] = NULL
        assert call(qc, f, *args) == qc.QC_ERR_ARG, pos
    for pos in (0, 1, 7, 8, 9):
        args = list(ok)
        args[pos] = MIS
        assert call(qc, f, *args) == qc.QC_ERR_ALIGN, pos
    assert call(qc, f, NULL, NULL, 0, 256, 4, 7, 8, NULL, NULL, NULL, None) == qc.QC_OK


def test_encode_ternary_errors(qc):
    f = "qc_encode_ternary"
    ok = (A, A, 1000, 512, 3, 4, A, A, None)
    assert call(qc, f, *ok[:5], 2, *ok[6:]) == qc.QC_ERR_ARG  # offset % 4
    assert call(qc, f, A, A, -5, 512, 3, 4, A, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, A, 1000, 48, 3, 4, A, A, None) == qc.QC_ERR_ARG
    for pos in (0, 6, 7):
        args = list(ok)
        args[pos] = NULL
        assert call(qc, f, *args) == qc.QC_ERR_ARG, pos
    for pos in (0, 1, 6, 7):
        args = list(ok)
        args[pos] = MIS
        assert call(qc, f, *args) == qc.QC_ERR_ALIGN, pos
    assert call(qc, f, NULL, NULL, 0, 512, 3, 4, NULL, NULL, None) == qc.QC_OK


def test_encode_fp8_errors(qc):
    f = "qc_encode_fp8_rowwise"
    assert call(qc, f, A, -1, 128, A, A, None) == qc.QC_ERR_ARG
    for dim in (0, 2, 6, 130, 65540):
        assert call(qc, f, A, 10, dim, A, A, None) == qc.QC_ERR_UNSUPPORTED, dim
    assert call(qc, f, NULL, 10, 128, A, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, 10, 128, NULL, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, 10, 128, A, NULL, None) == qc.QC_ERR_ARG
    assert call(qc, f, MIS, 10, 128, A, A, None) == qc.QC_ERR_ALIGN
    assert call(qc, f, A, 10, 128, MIS, A, None) == qc.QC_ERR_ALIGN
    assert call(qc, f, NULL, 0, 128, NULL, NULL, None) == qc.QC_OK


def test_encode_qsgd_errors(qc):
    f = "qc_encode_qsgd"
    assert call(qc, f, A, A, 1000, 512, 16, 1, 2, A, A, None) == qc.QC_ERR_ARG  # offset % 4
    assert call(qc, f, A, A, 1000, 500, 16, 1, 0, A, A, None) == qc.QC_ERR_ARG
    for lv in (2, 4, 8, 15, 32):
        assert call(qc, f, A, A, 1000, 512, lv, 1, 0, A, A, None) == qc.QC_ERR_UNSUPPORTED
    assert call(qc, f, A, A, 1000, 512, 16, 1, 0, NULL, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, MIS, 1000, 512, 16, 1, 0, A, A, None) == qc.QC_ERR_ALIGN
    assert call(qc, f, NULL, NULL, 0, 512, 16, 1, 0, NULL, NULL, None) == qc.QC_OK


def test_encode_sign_errors(qc):
    f = "qc_encode_sign"
    assert call(qc, f, A, 2, A, 1000, 4096, A, A, None) == qc.QC_ERR_ARG  # xtype
    assert call(qc, f, A, 1, A, 1000, 4095, A, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, 1, A, 1000, 4096, A, NULL, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, 1, A, 1000, 4096, MIS, A, None) == qc.QC_ERR_ALIGN
    assert call(qc, f, NULL, 1, NULL, 0, 4096, NULL, NULL, None) == qc.QC_OK


def test_decode_errors(qc):
    f = "qc_decode"
    assert call(qc, f, 7, A, A, A, 100, 64, 8, A, None) == qc.QC_ERR_UNSUPPORTED
    assert call(qc, f, qc.QC_UNIFORM, A, A, A, 100, 64, 3, A, None) == qc.QC_ERR_UNSUPPORTED
    assert call(qc, f, qc.QC_TERNARY, A, A, NULL, 100, 64, 4, A, None) == qc.QC_ERR_UNSUPPORTED
    assert call(qc, f, qc.QC_TERNARY, A, A, NULL, 100, 96, 2, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, qc.QC_TERNARY, A, MIS, NULL, 100, 64, 2, A, None) == qc.QC_ERR_ALIGN
    assert call(qc, f, qc.QC_UNIFORM, A, A, NULL, 100, 64, 8, A, None) == qc.QC_ERR_ARG  # zero needed
    assert call(qc, f, qc.QC_FP8_ROWWISE, A, A, NULL, 100, 128, 8, A, None) == qc.QC_ERR_ARG  # n % dim
    assert call(qc, f, qc.QC_FP8_ROWWISE, A, A, NULL, 128, 6, 8, A, None) == qc.QC_ERR_UNSUPPORTED
    assert call(qc, f, qc.QC_QSGD, A, A, NULL, 100, 512, 4, A, None) == qc.QC_ERR_UNSUPPORTED
    assert call(qc, f, qc.QC_SIGN, A, A, NULL, 100, 512, 8, A, None) == qc.QC_ERR_UNSUPPORTED
    assert call(qc, f, qc.QC_SIGN, A, A, NULL, 100, 300, 1, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, qc.QC_SIGN, A, A, NULL, 100, 512, 1, MIS, None) == qc.QC_ERR_ALIGN
    assert call(qc, f, qc.QC_SIGN, NULL, NULL, NULL, 0, 512, 1, NULL, None) == qc.QC_OK


def test_dequant_accumulate_errors(qc):
    f = "qc_dequant_accumulate"
    U = qc.QC_UNIFORM
    assert call(qc, f, U, A, A, A, 0, 100, 64, 8, A, 0, NULL, NULL, NULL, None) == qc.QC_ERR_ARG
    assert call(qc, f, U, A, A, A, 65536, 100, 64, 8, A, 0, NULL, NULL, NULL, None) == qc.QC_ERR_ARG
    assert call(qc, f, U, A, A, A, 4, 100, 64, 8, A, 0, A, NULL, NULL, None) == qc.QC_ERR_ARG
    assert call(qc, f, qc.QC_SIGN, A, A, NULL, 4, 100, 64, 1, A, 0, A, A, A, None) == qc.QC_ERR_UNSUPPORTED
    assert call(qc, f, qc.QC_TERNARY, A, A, NULL, 4, 100, 64, 2, A, 0, A, A, A, None) == qc.QC_ERR_UNSUPPORTED
    assert call(qc, f, U, A, A, A, 4, 100, 64, 3, A, 0, NULL, NULL, NULL, None) == qc.QC_ERR_UNSUPPORTED
    assert call(qc, f, qc.QC_FP8_ROWWISE, A, A, NULL, 4, 96 * 3, 96, 8, A, 0, NULL, NULL, NULL,
                None) == qc.QC_ERR_UNSUPPORTED  # rows for accumulation: power-of-two dims
    assert call(qc, f, U, A, A, A, 4, 100, 64, 8, MIS, 0, NULL, NULL, NULL, None) == qc.QC_ERR_ALIGN
    assert call(qc, f, U, A, A, A, 4, 100, 64, 8, A, 0, A, A, MIS, None) == qc.QC_ERR_ALIGN
    assert call(qc, f, U, NULL, NULL, NULL, 4, 0, 64, 8, NULL, 0, NULL, NULL, NULL, None) == qc.QC_OK


def test_shared_scale_errors(qc):
    f = "qc_bucket_absmax"
    assert call(qc, f, A, A, -1, 512, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, A, 100, 500, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, NULL, A, 100, 512, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, A, 100, 512, NULL, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, MIS, 100, 512, A, None) == qc.QC_ERR_ALIGN
    assert call(qc, f, NULL, NULL, 0, 512, NULL, None) == qc.QC_OK
    f = "qc_absmax_combine"
    assert call(qc, f, A, 0, 10, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, 65536, 10, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, 2, -1, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, NULL, 2, 10, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, 2, 10, MIS, None) == qc.QC_ERR_ALIGN
    assert call(qc, f, NULL, 2, 0, NULL, None) == qc.QC_OK
    f = "qc_encode_int8_shared"
    ok = (A, A, 1000, 512, A, A, A, None)
    for pos in (0, 4, 5, 6):
        args = list(ok)
        args[pos] = NULL
        assert call(qc, f, *args) == qc.QC_ERR_ARG, pos
    for pos in (0, 1, 4, 5, 6):
        args = list(ok)
        args[pos] = MIS
        assert call(qc, f, *args) == qc.QC_ERR_ALIGN, pos
    assert call(qc, f, A, A, 1000, 96, A, A, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, NULL, NULL, 0, 512, NULL, NULL, NULL, None) == qc.QC_OK
    f = "qc_sum_int8_shared"
    assert call(qc, f, A, 0, 100, 512, A, A, 0, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, 3, 100, 512, A, NULL, 0, NULL, None) == qc.QC_ERR_ARG   # no output
    assert call(qc, f, A, 3, 100, 512, A, NULL, 1, A, None) == qc.QC_ERR_ARG      # accumulate needs isum
    assert call(qc, f, A, 3, 100, 512, NULL, A, 0, A, None) == qc.QC_ERR_ARG      # out needs scale
    assert call(qc, f, NULL, 3, 100, 512, A, A, 0, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, 3, 100, 512, A, MIS, 0, A, None) == qc.QC_ERR_ALIGN
    assert call(qc, f, NULL, 3, 0, 512, NULL, A, 0, NULL, None) == qc.QC_OK
    # the fp32 accumulator does not take shared-scale payloads
    assert call(qc, "qc_dequant_accumulate", qc.QC_INT8_SHARED, A, A, NULL, 4, 100, 64, 8, A, 0, NULL, NULL,
                NULL, None) == qc.QC_ERR_UNSUPPORTED


def test_majority_vote_errors(qc):
    f = "qc_majority_vote"
    assert call(qc, f, A, 0, 100, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, 70000, 100, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, NULL, 3, 100, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, 3, 100, MIS, None) == qc.QC_ERR_ALIGN
    assert call(qc, f, NULL, 3, 0, NULL, None) == qc.QC_OK


def test_binding_rejects_undersized_buffers_before_the_library(qc):
    """The Python binding checks tensor capacities; CPU tensors are refused
    outright (these raise before any library call)."""
    import torch

    x = torch.zeros(10)
    with pytest.raises(ValueError):
        qc.qc_encode_uniform(x, None, 10, 64, 8, x, x, x, stream=0)


def test_tensor_index_plan(qc):
    """The bucket plan qc_tensor_index builds on the host: prefix offsets,
    and for each 4096-element segment the tensor holding its first element
    (empty tensors skipped), checked against numpy's searchsorted."""
    import numpy as np

    rng = np.random.default_rng(0)
    shift = qc.QC_INDEX_SHIFT
    for sizes in ([5], [0, 0, 7, 0], [4096, 4096], [4095, 1, 0, 8192, 3],
                  list(rng.integers(0, 9000, 300)), list(rng.integers(0, 3, 5000))):
        sizes = np.array(sizes, dtype=np.int64)
        n = int(sizes.sum())
        offs = np.empty(sizes.size + 1, np.int64)
        nseg = -(-n // (1 << shift))
        seg = np.empty(nseg + 1, np.int32)
        qc.qc_tensor_index(sizes, sizes.size, offs, seg)
        assert offs[0] == 0 and np.array_equal(np.diff(offs), sizes)
        for j in range(nseg + 1):
            g = max(0, min(j << shift, n - 1))
            t = int(np.searchsorted(offs, g, side="right")) - 1
            t = min(t, sizes.size - 1)
            if n > 0:
                assert offs[seg[j]] <= g < offs[seg[j] + 1], (j, g, seg[j])
                assert seg[j] == t
    # a rejected plan writes nothing: a negative size after a valid one, and
    # sizes whose total would pass 2^56 elements
    for bad in (np.array([3, -1], np.int64), np.array([5, 1 << 55, 1 << 55, 7], np.int64)):
        offs = np.full(bad.size + 1, -77, np.int64)
        seg = np.full(8, -77, np.int32)
        with pytest.raises(qc.QcError):
            qc.qc_tensor_index(bad, bad.size, offs, seg)
        assert np.all(offs == -77) and np.all(seg == -77)


def test_multi_entry_point_errors(qc):
    f = "qc_encode_uniform_multi"
    ok = (A, A, A, 5, 1000, A, 512, 8, A, A, A, None)
    for pos in (0, 1, 2, 8, 9, 10):
        args = list(ok)
        args[pos] = NULL
        assert call(qc, f, *args) == qc.QC_ERR_ARG, pos
    args = list(ok)
    args[3] = 0
    assert call(qc, f, *args) == qc.QC_ERR_ARG
    args = list(ok)
    args[7] = 3
    assert call(qc, f, *args) == qc.QC_ERR_UNSUPPORTED
    args = list(ok)
    args[6] = 65536   # above QC_MAX_LIST_BUCKET
    assert call(qc, f, *args) == qc.QC_ERR_UNSUPPORTED
    for pos, bad in ((0, A + 4), (1, A + 4), (2, A + 2), (5, MIS), (8, MIS)):
        args = list(ok)
        args[pos] = bad
        assert call(qc, f, *args) == qc.QC_ERR_ALIGN, pos
    f = "qc_decode_multi"
    ok = (0, A, A, A, 1000, 512, 8, A, A, A, 5, None)
    for pos in (7, 8, 9):
        args = list(ok)
        args[pos] = NULL
        assert call(qc, f, *args) == qc.QC_ERR_ARG, pos
    args = list(ok)
    args[10] = 0
    assert call(qc, f, *args) == qc.QC_ERR_ARG
    args = list(ok)
    args[9] = A + 2
    assert call(qc, f, *args) == qc.QC_ERR_ALIGN


# The other encoders' list forms: (name, valid arguments, positions of
# required pointers, position of the bucket, positions of 16-byte aligned
# outputs).  The list tables sit at positions 0-2 (0, 2, 3 for sign).
LIST_CALLS = [
    ("qc_encode_uniform_stochastic_multi", (A, A, A, 5, 1000, A, 512, 4, 7, 0, A, A, A, None), (10, 11, 12), 6,
     (5, 10)),
    ("qc_encode_qsgd_multi", (A, A, A, 5, 1000, A, 512, 16, 7, 0, A, A, None), (10, 11), 6, (5, 10)),
    ("qc_encode_ternary_multi", (A, A, A, 5, 1000, A, 512, 7, 0, A, A, None), (9, 10), 6, (5, 9)),
    ("qc_encode_sign_multi", (A, 1, A, A, 5, 1000, A, 512, A, A, None), (8, 9), 7, (6, 8)),
    ("qc_bucket_absmax_multi", (A, A, A, 5, 1000, A, 512, A, None), (7,), 6, (5, 7)),
    ("qc_encode_int8_shared_multi", (A, A, A, 5, 1000, A, 512, A, A, A, None), (7, 8, 9), 6, (5, 8)),
]


@pytest.mark.parametrize("name,ok,required,bpos,aligned", LIST_CALLS, ids=[c[0] for c in LIST_CALLS])
def test_list_encoders_errors(qc, name, ok, required, bpos, aligned):
    tables = (0, 2, 3) if name == "qc_encode_sign_multi" else (0, 1, 2)
    for pos in tables + required:
        args = list(ok)
        args[pos] = NULL
        assert call(qc, name, *args) == qc.QC_ERR_ARG, pos
    for bucket, st in ((65536, qc.QC_ERR_UNSUPPORTED), (100, qc.QC_ERR_ARG), (32, qc.QC_ERR_ARG)):
        args = list(ok)
        args[bpos] = bucket
        assert call(qc, name, *args) == st, bucket
    for pos in aligned:
        args = list(ok)
        args[pos] = MIS
        assert call(qc, name, *args) == qc.QC_ERR_ALIGN, pos
    args = list(ok)
    args[tables[0]] = A + 4  # the pointer table must be 8-byte aligned
    assert call(qc, name, *args) == qc.QC_ERR_ALIGN
    # an empty list call is valid and does nothing, whatever the pointers
    args = list(ok)
    args[bpos - 2] = 0
    for pos in required:
        args[pos] = NULL
    assert call(qc, name, *args) == qc.QC_OK


def test_topk_errors(qc):
    f = "qc_encode_topk"
    ok = (A, A, 1000, 512, 8, A, A, None)
    for k in (0, -1, 513):
        assert call(qc, f, A, A, 1000, 512, k, A, A, None) == qc.QC_ERR_ARG, k
    assert call(qc, f, A, A, 1000, 500, 8, A, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, A, 100000, 131072, 8, A, A, None) == qc.QC_ERR_ARG
    for pos in (0, 5, 6):
        args = list(ok)
        args[pos] = NULL
        assert call(qc, f, *args) == qc.QC_ERR_ARG, pos
    for pos, bad in ((0, MIS), (1, MIS), (5, A + 2), (6, A + 1)):
        args = list(ok)
        args[pos] = bad
        assert call(qc, f, *args) == qc.QC_ERR_ALIGN, pos
    assert call(qc, f, NULL, NULL, 0, 512, 8, NULL, NULL, None) == qc.QC_OK
    f = "qc_encode_topk_multi"
    ok = (A, A, A, 5, 1000, A, 512, 8, A, A, None)
    for pos in (0, 1, 2, 8, 9):
        args = list(ok)
        args[pos] = NULL
        assert call(qc, f, *args) == qc.QC_ERR_ARG, pos
    for k in (0, 513):
        args = list(ok)
        args[7] = k
        assert call(qc, f, *args) == qc.QC_ERR_ARG, k
    for bucket in (100, 32, 131072):
        args = list(ok)
        args[6] = bucket
        assert call(qc, f, *args) == qc.QC_ERR_ARG, bucket
    for pos, bad in ((0, A + 4), (1, A + 4), (2, A + 2), (5, MIS), (8, A + 2), (9, A + 1)):
        args = list(ok)
        args[pos] = bad
        assert call(qc, f, *args) == qc.QC_ERR_ALIGN, pos
    assert call(qc, f, A, A, A, 5, 0, NULL, 512, 8, NULL, NULL, None) == qc.QC_OK
    f = "qc_decode_topk"
    assert call(qc, f, A, A, 1000, 512, 600, A, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, A, 1000, 512, 8, NULL, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, A, 1000, 512, 8, MIS, None) == qc.QC_ERR_ALIGN
    f = "qc_topk_accumulate"
    assert call(qc, f, A, A, 0, 1000, 512, 8, A, 0, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, A, 3, 1000, 512, 8, NULL, 0, None) == qc.QC_ERR_ARG
    assert call(qc, f, A, A, 3, 1000, 512, 8, MIS, 0, None) == qc.QC_ERR_ALIGN
    assert call(qc, f, NULL, NULL, 3, 0, 512, 8, NULL, 0, None) == qc.QC_OK


def test_missing_library_fails_loudly():
    """No CPU fallback: with libqc.so absent, the first call raises instead of
    computing anything on the host."""
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import embedding_communication_codecs_amd.binding as b\n"
        "b.LIB_PATH = '/nonexistent/libqc.so'\n"
        "try:\n"
        "    b.qc_payload_bytes(0, 1024, 64, 8)\n"
        "except RuntimeError as e:\n"
        "    print('raised', 'missing' in str(e))\n"
        "else:\n"
        "    print('returned')\n" % ROOT
    )
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.stdout.strip() == "raised True", r.stdout + r.stderr
