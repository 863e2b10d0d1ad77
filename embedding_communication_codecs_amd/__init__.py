"""Quantized-communication codec for MI355X (gfx950).

The codec sits between a training framework and a collective: it encodes
gradients and embedding-lookup payloads into compact wire formats with
fused error feedback, decodes them, and aggregates many workers' payloads on
the receive side.  The work runs in hand-written HIP kernels behind the C
ABI declared in include/qc.h (built into libqc.so by ``build.py``); the
``binding`` module exposes the same entry points to Python.
"""
from .binding import (  # noqa: F401
    EXPORTS,
    QC_BF16,
    QC_ERR_ALIGN,
    QC_ERR_ARG,
    QC_ERR_LAUNCH,
    QC_ERR_UNSUPPORTED,
    QC_F32,
    QC_FP8_ROWWISE,
    QC_INDEX_SHIFT,
    QC_INT8_SHARED,
    QC_MAX_BUCKET,
    QC_MAX_TOPK_BUCKET,
    QC_MAX_WORKERS,
    QC_MIN_BUCKET,
    QC_OK,
    QC_QSGD,
    QC_SIGN,
    QC_TERNARY,
    QC_UNIFORM,
    QcError,
    TensorTable,
    lib,
    nbuckets,
    payload_bytes,
    qc_absmax_combine,
    qc_bucket_absmax,
    qc_decode,
    qc_decode_multi,
    qc_decode_topk,
    qc_dequant_accumulate,
    qc_encode_fp8_rowwise,
    qc_encode_int8_shared,
    qc_encode_qsgd,
    qc_encode_sign,
    qc_encode_ternary,
    qc_encode_topk,
    qc_encode_uniform,
    qc_encode_uniform_stochastic,
    qc_encode_uniform_multi,
    qc_majority_vote,
    qc_payload_bytes,
    qc_status_str,
    qc_sum_int8_shared,
    qc_tensor_index,
    qc_topk_accumulate,
)
