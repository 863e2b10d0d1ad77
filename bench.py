"""Benchmark of the quantized-communication codec on one MI355X.

One step is one pass of the whole codec hot path over one batch of
synthetic input, every op at its full workload size:

  uniform INT8 + error feedback, 65,536 fp32 (buckets of 4,096), and decode
  rowwise FP8-E4M3 encode of 1,000,000 x 128 fp32 embedding rows, and decode
  QSGD + error feedback, 1e9 fp32 (buckets of 512, Philox rounding), and decode
  1-bit sign + error feedback, 2^28 bf16 (buckets of 4,096), and decode
  majority vote over 16 sign payloads of 2^28 bits
  dequantize-accumulate of 64 INT8 payloads of 2^26 (buckets of 2,048)
    with the sum requantized to INT8 in the same pass

Beside the step, in a timed region of its own that `value` does not
include, the low-bit extensions run on the same 1e9-element gradient:
2-bit uniform and 4-bit stochastic uniform (buckets of 512, error
feedback), TernGrad (buckets of 512, error feedback), shared-scale INT8
(the per-bucket max statistic and the encode with an agreed maximum, error
feedback), their decoders, and the receive-side sums of 64 workers'
payloads of 2^26: TernGrad, 2-bit (requantized to 2 bits in the same
pass) and shared-scale INT8 (an exact integer sum, dequantized once); and
the bucketing front-end on the parameter list of a 24-layer, width-1024
transformer (288 tensors, 302M fp32): INT8 + EF of the whole list in one
launch, the same tensors encoded one launch per tensor, and the decode back
into the list; top-k sparsification (4 of every 4,096 coordinates, error
feedback) of the 1e9 gradient, its decode, and the sum of 64 workers'
top-k payloads of 2^26.  They are reported
under `extensions`, in the same form as `ops`.

Encoders run first and decoders later in the step, so a decoder never
reads a payload that is still in the 256 MB last-level cache.  Inputs are
generated on the GPU (seeded) before timing; the timed region only runs
the kernels.

Printed: one JSON line.  `value` is codec throughput in GB/s of logical
input (fp32 bytes of each encoded/decoded tensor, bf16 bytes for the sign
encoder's input, m*n*4 for the accumulation, packed bits for the vote)
summed over the step and divided by the step time.  `ops` gives each op's
time, its input GB/s and its algorithmic HBM GB/s against the 8 TB/s peak;
`roofline` is that figure for the op with the largest time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
CSRC = os.path.join(ROOT, "embedding_communication_codecs_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic_codec_suite.json")

# workload sizes
C1_N, C1_B = 65536, 4096
C2_ROWS, C2_DIM = 1_000_000, 128
C3_N, C3_B = 1_000_000_000, 512
C4_N, C4_B, C4_M = 1 << 28, 4096, 16
C5_M, C5_N, C5_B = 64, 1 << 26, 2048
# low-bit extensions: on the QSGD gradient, and 64 workers' payloads like C5
X_N, X_B = C3_N, 512
X_M, X_AN, X_AB = 64, 1 << 26, 2048
# bucketing front-end: the parameter list of a 24-layer transformer with
# width 1024 (per layer: qkv weight and bias, output projection weight and
# bias, two layer norms' weight and bias, two MLP weights and biases)
T_D, T_L, T_B = 1024, 24, 4096
# top-k: density about 1/1000 (4 of every 4,096 coordinates)
K_B, K_K = 4096, 4


def tensor_list_sizes():
    d = T_D
    layer = [3 * d * d, 3 * d, d * d, d, d, d, 4 * d * d, 4 * d, 4 * d * d, d, d, d]
    return layer * T_L


# The kernel source each op runs (plus the shared headers below): counter
# traffic taken for an op stays valid while these files are unchanged.
SHARED_SOURCES = ["qc_device.hpp", "qc_bucket.hpp", "qc_launch.hpp", "../../include/qc.h"]
OP_SOURCE = {
    **{o: "k_encode.hpp" for o in ("uniform_enc", "qsgd_enc", "sign_enc", "int2_enc", "stoch4_enc", "tern_enc",
                                   "shared_absmax", "shared_enc", "list_enc", "list_enc_per_tensor")},
    "fp8_enc": "k_fp8.hip",
    **{o: "k_decode.hip" for o in ("uniform_dec", "fp8_dec", "qsgd_dec", "sign_dec", "int2_dec", "tern_dec",
                                   "list_dec")},
    **{o: "k_accumulate.hip" for o in ("acc_requant", "acc_tern", "acc_int2_requant")},
    "sign_vote": "k_vote.hip",
    "shared_sum": "k_shared_sum.hip",
    **{o: "k_topk.hip" for o in ("topk_enc", "topk_dec", "topk_sum")},
}


def source_hash(op: str) -> str:
    h = hashlib.sha256()
    for f in [OP_SOURCE[op]] + SHARED_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def op_bytes():
    """(logical input bytes, algorithmic HBM bytes read+written) per op."""
    nb1 = -(-C1_N // C1_B)
    n2 = C2_ROWS * C2_DIM
    nb3 = -(-C3_N // C3_B)
    nb4 = -(-C4_N // C4_B)
    nb5 = C5_N // C5_B
    sign_pb = -(-C4_N // 32) * 4
    return {
        # x + ef read, ef written, codes + scale/zero written
        "uniform_enc": (4 * C1_N, 4 * C1_N * 3 + C1_N + 8 * nb1),
        "uniform_dec": (4 * C1_N, C1_N + 8 * nb1 + 4 * C1_N),
        "fp8_enc": (4 * n2, 4 * n2 + n2 + 4 * C2_ROWS),
        "fp8_dec": (4 * n2, n2 + 4 * C2_ROWS + 4 * n2),
        "qsgd_enc": (4 * C3_N, 12 * C3_N + C3_N // 2 + 4 * nb3),
        "qsgd_dec": (4 * C3_N, C3_N // 2 + 4 * nb3 + 4 * C3_N),
        "sign_enc": (2 * C4_N, 2 * C4_N + 8 * C4_N + sign_pb + 4 * nb4),
        "sign_vote": (C4_M * sign_pb, C4_M * sign_pb + sign_pb),
        "sign_dec": (4 * C4_N, sign_pb + 4 * nb4 + 4 * C4_N),
        "acc_requant": (4 * C5_M * C5_N, C5_M * (C5_N + 8 * nb5) + 4 * C5_N + C5_N + 8 * nb5),
        **ext_bytes(),
    }


def ext_bytes():
    nbx = -(-X_N // X_B)
    nba = X_AN // X_AB
    return {
        # x + ef read, ef written, 2-bit codes + scale/zero written
        "int2_enc": (4 * X_N, 12 * X_N + X_N // 4 + 8 * nbx),
        "stoch4_enc": (4 * X_N, 12 * X_N + X_N // 2 + 8 * nbx),
        "tern_enc": (4 * X_N, 12 * X_N + X_N // 4 + 4 * nbx),
        "int2_dec": (4 * X_N, X_N // 4 + 8 * nbx + 4 * X_N),
        "tern_dec": (4 * X_N, X_N // 4 + 4 * nbx + 4 * X_N),
        "acc_tern": (4 * X_M * X_AN, X_M * (X_AN // 4 + 4 * nba) + 4 * X_AN),
        "acc_int2_requant": (4 * X_M * X_AN, X_M * (X_AN // 4 + 8 * nba) + 4 * X_AN + X_AN // 4 + 8 * nba),
        # shared-scale INT8: the local statistic (x + ef read), the encode
        # with the agreed maximum, and the exact integer sum of 64 workers
        "shared_absmax": (4 * X_N, 8 * X_N + 4 * nbx),
        "shared_enc": (4 * X_N, 12 * X_N + X_N + 8 * nbx),
        "shared_sum": (4 * X_M * X_AN, X_M * X_AN + 4 * X_AN + 4 * nba),
        **list_bytes(),
        **topk_bytes(),
    }


def topk_bytes():
    pairs = 8 * K_K * -(-X_N // K_B)
    pairs_w = 8 * K_K * (X_AN // K_B)
    return {
        # x + ef read, ef written, (index, value) pairs written
        "topk_enc": (4 * X_N, 12 * X_N + pairs),
        # pairs read, the dense vector written (zeros and values)
        "topk_dec": (4 * X_N, pairs + 4 * X_N),
        # 64 workers' pairs read, the dense sum written once
        "topk_sum": (4 * X_M * X_AN, X_M * pairs_w + 4 * X_AN),
    }


def list_bytes():
    sizes = tensor_list_sizes()
    n = sum(sizes)
    nb = -(-n // T_B)
    nb_pt = sum(-(-s // T_B) for s in sizes)
    return {
        # x + ef read, ef written, INT8 codes + scale/zero written
        "list_enc": (4 * n, 13 * n + 8 * nb),
        "list_enc_per_tensor": (4 * n, 13 * n + 8 * nb_pt),
        "list_dec": (4 * n, n + 8 * nb + 4 * n),
    }


ORDER = ["uniform_enc", "qsgd_enc", "fp8_enc", "sign_enc", "acc_requant", "sign_vote", "qsgd_dec",
         "fp8_dec", "sign_dec", "uniform_dec"]
EXT_ORDER = ["int2_enc", "stoch4_enc", "tern_enc", "shared_absmax", "shared_enc", "acc_tern", "acc_int2_requant",
             "shared_sum", "int2_dec", "tern_dec", "list_enc", "list_enc_per_tensor", "list_dec",
             "topk_enc", "topk_sum", "topk_dec"]


# ------------------------------------------------------------- GPU setup


def setup(qc, synth, torch, ext):
    dev = torch.device("cuda")
    st = {}
    U8, F32 = torch.uint8, torch.float32

    def empty(nbytes):
        return torch.empty(nbytes, dtype=U8, device=dev)

    # C1
    st["c1_x"] = synth.device_normal(C1_N, 1e-3, 1001, dev)
    st["c1_ef"] = torch.zeros(C1_N, dtype=F32, device=dev)
    st["c1_codes"] = empty(qc.payload_bytes(qc.QC_UNIFORM, C1_N, C1_B, 8))
    st["c1_scale"] = torch.empty(C1_N // C1_B, dtype=F32, device=dev)
    st["c1_zero"] = torch.empty(C1_N // C1_B, dtype=F32, device=dev)
    st["c1_out"] = torch.empty(C1_N, dtype=F32, device=dev)
    # C2
    st["c2_x"] = synth.device_embedding_rows(C2_ROWS, C2_DIM, 0.05, 0.001, 50.0, 2001, dev)
    st["c2_codes"] = empty(qc.payload_bytes(qc.QC_FP8_ROWWISE, C2_ROWS * C2_DIM, C2_DIM, 8))
    st["c2_scale"] = torch.empty(C2_ROWS, dtype=F32, device=dev)
    st["c2_out"] = torch.empty(C2_ROWS * C2_DIM, dtype=F32, device=dev)
    # C3
    st["c3_x"] = synth.device_laplace(C3_N, 1e-4, 3001, dev)
    st["c3_ef"] = torch.zeros(C3_N, dtype=F32, device=dev)
    st["c3_words"] = empty(qc.payload_bytes(qc.QC_QSGD, C3_N, C3_B, 16))
    st["c3_norm"] = torch.empty(-(-C3_N // C3_B), dtype=F32, device=dev)
    st["c3_out"] = torch.empty(C3_N, dtype=F32, device=dev)
    # C4
    st["c4_x"] = synth.device_bf16_normal(C4_N, 1e-3, 4001, dev)
    st["c4_ef"] = torch.zeros(C4_N, dtype=F32, device=dev)
    pb4 = qc.payload_bytes(qc.QC_SIGN, C4_N, C4_B, 1)
    st["c4_words"] = empty(pb4)
    st["c4_scale"] = torch.empty(C4_N // C4_B, dtype=F32, device=dev)
    st["c4_arena"] = synth.device_words(C4_M * pb4 // 4, 4100, dev)
    st["c4_vote"] = empty(pb4)
    st["c4_out"] = torch.empty(C4_N, dtype=F32, device=dev)
    # C5: 64 workers' INT8 payloads, encoded from outlier gradients
    pb5 = qc.payload_bytes(qc.QC_UNIFORM, C5_N, C5_B, 8)
    nb5 = C5_N // C5_B
    st["c5_arena"] = empty(C5_M * pb5)
    st["c5_scale"] = torch.empty(C5_M * nb5, dtype=F32, device=dev)
    st["c5_zero"] = torch.empty(C5_M * nb5, dtype=F32, device=dev)
    for w in range(C5_M):
        g = synth.device_outlier_grad(C5_N, 1e-3, 0.01, 100.0, 5000 + w, dev)
        qc.qc_encode_uniform(g, None, C5_N, C5_B, 8, st["c5_arena"][w * pb5:(w + 1) * pb5],
                             st["c5_scale"][w * nb5:(w + 1) * nb5], st["c5_zero"][w * nb5:(w + 1) * nb5])
        del g
    st["c5_acc"] = torch.empty(C5_N, dtype=F32, device=dev)
    st["c5_rq"] = empty(pb5)
    st["c5_rqs"] = torch.empty(nb5, dtype=F32, device=dev)
    st["c5_rqz"] = torch.empty(nb5, dtype=F32, device=dev)
    if ext:
        setup_ext(qc, synth, torch, st, empty)
    torch.cuda.synchronize()
    return st


def setup_ext(qc, synth, torch, st, empty):
    dev, F32 = torch.device("cuda"), torch.float32
    nbx = -(-X_N // X_B)
    st["x_ef"] = torch.zeros(X_N, dtype=F32, device=dev)
    st["x_i2"] = empty(qc.payload_bytes(qc.QC_UNIFORM, X_N, X_B, 2))
    st["x_s4"] = empty(qc.payload_bytes(qc.QC_UNIFORM, X_N, X_B, 4))
    st["x_t"] = empty(qc.payload_bytes(qc.QC_TERNARY, X_N, X_B, 2))
    for k in ("x_i2s", "x_i2z", "x_s4s", "x_s4z", "x_ts"):
        st[k] = torch.empty(nbx, dtype=F32, device=dev)
    # 64 workers' TernGrad and 2-bit payloads of outlier gradients
    nba = X_AN // X_AB
    pbt = qc.payload_bytes(qc.QC_TERNARY, X_AN, X_AB, 2)
    pbi = qc.payload_bytes(qc.QC_UNIFORM, X_AN, X_AB, 2)
    st["xa_t"], st["xa_i2"] = empty(X_M * pbt), empty(X_M * pbi)
    st["xa_ts"] = torch.empty(X_M * nba, dtype=F32, device=dev)
    st["xa_i2s"] = torch.empty(X_M * nba, dtype=F32, device=dev)
    st["xa_i2z"] = torch.empty(X_M * nba, dtype=F32, device=dev)
    for w in range(X_M):
        g = synth.device_outlier_grad(X_AN, 1e-3, 0.01, 100.0, 6000 + w, dev)
        sl = slice(w * nba, (w + 1) * nba)
        qc.qc_encode_ternary(g, None, X_AN, X_AB, 0x5445524E + w, 0, st["xa_t"][w * pbt:(w + 1) * pbt],
                             st["xa_ts"][sl])
        qc.qc_encode_uniform(g, None, X_AN, X_AB, 2, st["xa_i2"][w * pbi:(w + 1) * pbi], st["xa_i2s"][sl],
                             st["xa_i2z"][sl])
        del g
    # shared-scale INT8: every worker's bucket maxima, combined, then each
    # worker encodes with the agreed scale (its gradient drawn again)
    st["x_amax"] = torch.empty(nbx, dtype=F32, device=dev)
    st["x_i8s"] = empty(qc.payload_bytes(qc.QC_INT8_SHARED, X_N, X_B, 8))
    st["x_i8ss"] = torch.empty(nbx, dtype=F32, device=dev)
    qc.qc_bucket_absmax(st["c3_x"], None, X_N, X_B, st["x_amax"])
    pbs = qc.payload_bytes(qc.QC_INT8_SHARED, X_AN, X_AB, 8)
    stats = torch.empty(X_M * nba, dtype=F32, device=dev)
    for w in range(X_M):
        g = synth.device_outlier_grad(X_AN, 1e-3, 0.01, 100.0, 6000 + w, dev)
        qc.qc_bucket_absmax(g, None, X_AN, X_AB, stats[w * nba:(w + 1) * nba])
        del g
    st["xs_amax"] = torch.empty(nba, dtype=F32, device=dev)
    qc.qc_absmax_combine(stats, X_M, nba, st["xs_amax"])
    st["xs_codes"] = empty(X_M * pbs)
    st["xs_scale"] = torch.empty(nba, dtype=F32, device=dev)
    for w in range(X_M):
        g = synth.device_outlier_grad(X_AN, 1e-3, 0.01, 100.0, 6000 + w, dev)
        qc.qc_encode_int8_shared(g, None, X_AN, X_AB, st["xs_amax"], st["xs_codes"][w * pbs:(w + 1) * pbs],
                                 st["xs_scale"])
        del g
    # the transformer parameter list, as separate tensors (views of one
    # allocation would hide nothing: the kernel only sees pointers)
    sizes = tensor_list_sizes()
    st["tl_x"] = [synth.device_normal(sz, 1e-3, 7000 + k, dev) for k, sz in enumerate(sizes)]
    st["tl_table"] = qc.TensorTable(st["tl_x"])
    tn = st["tl_table"].n
    tnb = -(-tn // T_B)
    st["tl_ef"] = torch.zeros(tn, dtype=F32, device=dev)
    st["tl_codes"] = empty(qc.payload_bytes(qc.QC_UNIFORM, tn, T_B, 8))
    st["tl_scale"] = torch.empty(tnb, dtype=F32, device=dev)
    st["tl_zero"] = torch.empty(tnb, dtype=F32, device=dev)
    st["tl_out"] = [torch.empty(sz, dtype=F32, device=dev) for sz in sizes]
    st["tl_out_table"] = qc.TensorTable(st["tl_out"])
    # per-tensor encoding: each tensor its own payload, scales and residual
    st["tl_pt"] = []
    off = 0
    for k, sz in enumerate(sizes):
        nbk = -(-sz // T_B)
        st["tl_pt"].append((st["tl_x"][k], st["tl_ef"][off: off + sz], sz,
                            empty(qc.payload_bytes(qc.QC_UNIFORM, sz, T_B, 8)),
                            torch.empty(nbk, dtype=F32, device=dev), torch.empty(nbk, dtype=F32, device=dev)))
        off += sz
    # top-k payloads: the 1e9 gradient, and 64 workers of 2^26
    kslots = -(-X_N // K_B) * K_K
    st["k_vals"] = torch.empty(kslots, dtype=F32, device=dev)
    st["k_idx"] = torch.empty(kslots, dtype=torch.int32, device=dev)
    wslots = (X_AN // K_B) * K_K
    st["kw_vals"] = torch.empty(X_M * wslots, dtype=F32, device=dev)
    st["kw_idx"] = torch.empty(X_M * wslots, dtype=torch.int32, device=dev)
    for w in range(X_M):
        g = synth.device_outlier_grad(X_AN, 1e-3, 0.01, 100.0, 6000 + w, dev)
        qc.qc_encode_topk(g, None, X_AN, K_B, K_K, st["kw_vals"][w * wslots:(w + 1) * wslots],
                          st["kw_idx"][w * wslots:(w + 1) * wslots])
        del g
    st["xa_acc"] = torch.empty(X_AN, dtype=F32, device=dev)
    st["xa_rq"] = empty(pbi)
    st["xa_rqs"] = torch.empty(nba, dtype=F32, device=dev)
    st["xa_rqz"] = torch.empty(nba, dtype=F32, device=dev)


def make_ops(qc, st):
    s = st
    return {
        "uniform_enc": lambda: qc.qc_encode_uniform(s["c1_x"], s["c1_ef"], C1_N, C1_B, 8, s["c1_codes"],
                                                    s["c1_scale"], s["c1_zero"]),
        "uniform_dec": lambda: qc.qc_decode(qc.QC_UNIFORM, s["c1_codes"], s["c1_scale"], s["c1_zero"], C1_N,
                                            C1_B, 8, s["c1_out"]),
        "fp8_enc": lambda: qc.qc_encode_fp8_rowwise(s["c2_x"], C2_ROWS, C2_DIM, s["c2_codes"], s["c2_scale"]),
        "fp8_dec": lambda: qc.qc_decode(qc.QC_FP8_ROWWISE, s["c2_codes"], s["c2_scale"], None,
                                        C2_ROWS * C2_DIM, C2_DIM, 8, s["c2_out"]),
        "qsgd_enc": lambda: qc.qc_encode_qsgd(s["c3_x"], s["c3_ef"], C3_N, C3_B, 16, 0x5153474400000001, 0,
                                              s["c3_words"], s["c3_norm"]),
        "qsgd_dec": lambda: qc.qc_decode(qc.QC_QSGD, s["c3_words"], s["c3_norm"], None, C3_N, C3_B, 16,
                                         s["c3_out"]),
        "sign_enc": lambda: qc.qc_encode_sign(s["c4_x"], qc.QC_BF16, s["c4_ef"], C4_N, C4_B, s["c4_words"],
                                              s["c4_scale"]),
        "sign_vote": lambda: qc.qc_majority_vote(s["c4_arena"], C4_M, C4_N, s["c4_vote"]),
        "sign_dec": lambda: qc.qc_decode(qc.QC_SIGN, s["c4_words"], s["c4_scale"], None, C4_N, C4_B, 1,
                                         s["c4_out"]),
        "acc_requant": lambda: qc.qc_dequant_accumulate(qc.QC_UNIFORM, s["c5_arena"], s["c5_scale"],
                                                        s["c5_zero"], C5_M, C5_N, C5_B, 8, s["c5_acc"], False,
                                                        s["c5_rq"], s["c5_rqs"], s["c5_rqz"]),
        # extensions (present when setup_ext ran)
        "int2_enc": lambda: qc.qc_encode_uniform(s["c3_x"], s["x_ef"], X_N, X_B, 2, s["x_i2"], s["x_i2s"],
                                                 s["x_i2z"]),
        "stoch4_enc": lambda: qc.qc_encode_uniform_stochastic(s["c3_x"], s["x_ef"], X_N, X_B, 4, 0x53544F43, 0,
                                                              s["x_s4"], s["x_s4s"], s["x_s4z"]),
        "tern_enc": lambda: qc.qc_encode_ternary(s["c3_x"], s["x_ef"], X_N, X_B, 0x5445524E, 0, s["x_t"],
                                                 s["x_ts"]),
        "int2_dec": lambda: qc.qc_decode(qc.QC_UNIFORM, s["x_i2"], s["x_i2s"], s["x_i2z"], X_N, X_B, 2,
                                         s["c3_out"]),
        "tern_dec": lambda: qc.qc_decode(qc.QC_TERNARY, s["x_t"], s["x_ts"], None, X_N, X_B, 2, s["c3_out"]),
        "shared_absmax": lambda: qc.qc_bucket_absmax(s["c3_x"], s["x_ef"], X_N, X_B, s["x_amax"]),
        "shared_enc": lambda: qc.qc_encode_int8_shared(s["c3_x"], s["x_ef"], X_N, X_B, s["x_amax"], s["x_i8s"],
                                                       s["x_i8ss"]),
        "shared_sum": lambda: qc.qc_sum_int8_shared(s["xs_codes"], X_M, X_AN, X_AB, s["xs_scale"], None, False,
                                                    s["xa_acc"]),
        "list_enc": lambda: qc.qc_encode_uniform_multi(s["tl_table"].xs, s["tl_table"].offsets, s["tl_table"].seg_first,
                                                       s["tl_table"].ntensors,
                                                       s["tl_table"].n, s["tl_ef"], T_B, 8, s["tl_codes"],
                                                       s["tl_scale"], s["tl_zero"]),
        "list_enc_per_tensor": lambda: [qc.qc_encode_uniform(x, e, sz, T_B, 8, c, sc, z)
                                        for x, e, sz, c, sc, z in s["tl_pt"]],
        "list_dec": lambda: qc.qc_decode_multi(qc.QC_UNIFORM, s["tl_codes"], s["tl_scale"], s["tl_zero"],
                                               s["tl_table"].n, T_B, 8, s["tl_out_table"].xs,
                                               s["tl_out_table"].offsets, s["tl_out_table"].seg_first,
                                               s["tl_out_table"].ntensors),
        "topk_enc": lambda: qc.qc_encode_topk(s["c3_x"], s["x_ef"], X_N, K_B, K_K, s["k_vals"], s["k_idx"]),
        "topk_dec": lambda: qc.qc_decode_topk(s["k_vals"], s["k_idx"], X_N, K_B, K_K, s["c3_out"]),
        "topk_sum": lambda: qc.qc_topk_accumulate(s["kw_vals"], s["kw_idx"], X_M, X_AN, K_B, K_K, s["xa_acc"], False),
        "acc_tern": lambda: qc.qc_dequant_accumulate(qc.QC_TERNARY, s["xa_t"], s["xa_ts"], None, X_M, X_AN,
                                                     X_AB, 2, s["xa_acc"], False),
        "acc_int2_requant": lambda: qc.qc_dequant_accumulate(qc.QC_UNIFORM, s["xa_i2"], s["xa_i2s"], s["xa_i2z"],
                                                             X_M, X_AN, X_AB, 2, s["xa_acc"], False, s["xa_rq"],
                                                             s["xa_rqs"], s["xa_rqz"]),
    }


# ----------------------------------------------------------- cpu baseline


def host_cpu():
    """The host's logical CPU count and CPU model name."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return os.cpu_count(), model


def cpu_baseline():
    """The CPU oracle, single-threaded and pinned to one core, on a bounded
    sample of each op of the step: input GB/s per op (same input-byte
    accounting as the GPU figures) and over the whole sample."""
    import numpy as np

    import oracle as ora
    from embedding_communication_codecs_amd import synth

    ora.lib()
    ncpu, model = host_cpu()
    old_aff = os.sched_getaffinity(0)
    core = min(old_aff)
    os.sched_setaffinity(0, {core})
    per_op = {}

    def timed(op, in_bytes, sample, fn):
        t0 = time.perf_counter()
        r = fn()
        t = time.perf_counter() - t0
        per_op[op] = {"GBps": round(in_bytes / t / 1e9, 4), "s": round(t, 3), "input_bytes": in_bytes,
                      "sample": sample}
        return r

    try:
        # uniform (whole workload: it is small)
        g = synth.host_normal(C1_N, 1e-3, 1001)
        ef = np.zeros(C1_N, np.float32)
        p, s, z = timed("uniform_enc", 4 * C1_N, f"{C1_N} (whole)", lambda: ora.encode_uniform(g, ef, C1_B, 8))
        timed("uniform_dec", 4 * C1_N, f"{C1_N} (whole)", lambda: ora.decode_uniform(p, s, z, C1_N, C1_B, 8))
        # fp8: the whole 1,000,000 x 128 workload
        rows = C2_ROWS
        x = synth.host_embedding_rows(rows, C2_DIM, 0.05, 0.001, 50.0, 2001)
        p, s = timed("fp8_enc", 4 * rows * C2_DIM, f"{rows}x{C2_DIM} (whole)",
                     lambda: ora.encode_fp8_rowwise(x, rows, C2_DIM))
        timed("fp8_dec", 4 * rows * C2_DIM, f"{rows}x{C2_DIM} (whole)",
              lambda: ora.decode_fp8_rowwise(p, s, rows, C2_DIM))
        del x
        # qsgd: 2^27 elements
        n3 = 1 << 27
        x = synth.host_laplace(n3, 1e-4, 3001)
        ef = np.zeros(n3, np.float32)
        p, s = timed("qsgd_enc", 4 * n3, f"{n3} of {C3_N}",
                     lambda: ora.encode_qsgd(x, ef, C3_B, 0x5153474400000001, 0))
        timed("qsgd_dec", 4 * n3, f"{n3} of {C3_N}", lambda: ora.decode_qsgd(p, s, n3, C3_B))
        del x, ef
        # sign: 2^27 bf16, vote over 16 payloads of 2^27 bits, decode
        n4 = 1 << 27
        gb = synth.host_bf16_bits(synth.host_normal(n4, 1e-3, 4001))
        ef = np.zeros(n4, np.float32)
        p, s = timed("sign_enc", 2 * n4, f"{n4} of {C4_N}", lambda: ora.encode_sign(gb, ef, C4_B))
        pb = ora.payload_bytes(ora.SIGN, n4, 1)
        arena = np.concatenate([synth.host_words(pb // 4, 4100 + w).view(np.uint8) for w in range(C4_M)])
        timed("sign_vote", C4_M * pb, f"{C4_M}x{n4} bits of {C4_M}x{C4_N}",
              lambda: ora.majority_vote(arena, C4_M, n4))
        timed("sign_dec", 4 * n4, f"{n4} of {C4_N}", lambda: ora.decode_sign(p, s, n4, C4_B))
        del gb, ef, arena
        # accumulate: 64 workers x 2^22 elements, then requantize
        n5 = 1 << 22
        parts, scs, zes = [], [], []
        for w in range(C5_M):
            pp, ss, zz = ora.encode_uniform(synth.host_outlier_grad(n5, 1e-3, 0.01, 100.0, 5000 + w), None, C5_B, 8)
            parts.append(pp)
            scs.append(ss)
            zes.append(zz)
        arena, sc, ze = np.concatenate(parts), np.concatenate(scs), np.concatenate(zes)

        def acc_requant():
            acc = ora.dequant_accumulate(ora.UNIFORM, arena, sc, ze, C5_M, n5, C5_B, 8)
            return ora.encode_uniform(acc, None, C5_B, 8)

        timed("acc_requant", 4 * C5_M * n5, f"{C5_M}x{n5} of {C5_M}x{C5_N}", acc_requant)
    finally:
        os.sched_setaffinity(0, old_aff)
    total_in = sum(v["input_bytes"] for v in per_op.values())
    total_t = sum(v["s"] for v in per_op.values())
    return {
        "value": round(total_in / total_t / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "host_cpus": ncpu,
        "host_cpu_model": model,
        "pinned_core": core,
        "sample": ("every op of the step on a sample (per_op gives each): single-threaded C oracle pinned to one "
                   f"core of {ncpu}, same input-byte accounting as the GPU figures; {total_t:.1f} s of CPU time"),
        "per_op": per_op,
    }


def calibrate(torch, reps=10):
    """Achievable HBM rates of plain library kernels on 4 GiB buffers: a
    copy (read + write), a fill (write only) and a max-reduction (read
    only).  These are the practical ceilings the codec kernels are held to
    beside the 8 TB/s nominal peak."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)

    def avg_ms(fn):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    nbytes = 4 * n
    out = {
        "copy_GBps": round(2 * nbytes / avg_ms(lambda: b.copy_(a)) / 1e6, 1),
        "fill_GBps": round(nbytes / avg_ms(lambda: b.fill_(2.0)) / 1e6, 1),
        "read_GBps": round(nbytes / avg_ms(lambda: a.amax()) / 1e6, 1),
        "bytes": nbytes,
    }
    del a, b
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------ main


def load_traffic(kernel_op):
    """HBM bytes per launch measured with rocprofv3 counters for this op,
    if they were taken on the op's current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get("ops", {}).get(kernel_op)
    if e is None or e.get("source_hash") != source_hash(kernel_op):
        return None
    return e.get("hbm_bytes")


def time_ops(torch, ops, names, sizes, steps, warmup, extra):
    """Run `names` in order, `warmup` untimed passes then `steps` timed
    ones, with HIP events around every launch on the launching stream.
    Returns (wall ms per pass, per-op figures)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        for o in names:
            ops[o]()
        if extra:
            extra()
    torch.cuda.synchronize()
    ev = {o: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)] for o in names}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        for o in names:
            a, b = ev[o][k]
            a.record(stream)
            ops[o]()
            b.record(stream)
        if extra:
            extra()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    per_op = {}
    for o in names:
        ms = sum(a.elapsed_time(b) for a, b in ev[o]) / steps
        inb, hbm = sizes[o]
        per_op[o] = {
            "ms": round(ms, 4),
            "input_GBps": round(inb / (ms * 1e-3) / 1e9, 1),
            "hbm_GBps": round(hbm / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(hbm / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "algorithmic_bytes": hbm,
        }
    return wall_ms, per_op


def time_alone(torch, ops, names, sizes, per_op, reps):
    """Each op by itself: every launch starts on an idle GPU (synchronized
    before it), so its time does not depend on what ran before it in the
    step.  Adds ms_alone and hbm_frac_alone to per_op."""
    stream = torch.cuda.current_stream()
    for o in names:
        ops[o]()
        times = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            ops[o]()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        ms = sum(times) / reps
        hbm = sizes[o][1]
        per_op[o]["ms_alone"] = round(ms, 4)
        per_op[o]["hbm_frac_alone"] = round(hbm / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 200 steps keep the GPU busy for several seconds (about 1 s of the step,
    # 4 s of the extensions and 5 s of the ops timed alone), long enough for
    # an outside utilization sampler to see it
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ops", default=",".join(ORDER + EXT_ORDER), help="comma-separated subset of ops to run")
    ap.add_argument("--no-extensions", action="store_true", help="skip the low-bit extension ops")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy each step (counter calibration)")
    ap.add_argument("--calibrate", action="store_true",
                    help="only measure plain copy/fill/read bandwidth and print it")
    ap.add_argument("--no-alone", action="store_true",
                    help="skip timing each op alone (profiled runs keep only the timed passes)")
    ap.add_argument("--no-calibration", action="store_true", help="skip the copy/fill/read calibration")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the codec acts on one GPU's share of the payload and this "
              "build has no multi-GPU path; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import embedding_communication_codecs_amd as qc
    from embedding_communication_codecs_amd import synth

    qc.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate:
        print(json.dumps({"calibration": calibrate(torch)}))
        return
    wanted = args.ops.split(",")
    names = [o for o in ORDER if o in wanted]
    ext_names = [] if args.no_extensions else [o for o in EXT_ORDER if o in wanted]
    print(f"[bench] generating inputs for {names + ext_names}", file=sys.stderr, flush=True)
    st = setup(qc, synth, torch, bool(ext_names))
    ops = make_ops(qc, st)
    extra = None
    if args.copy_calibration:
        cal_src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        cal_dst = torch.empty_like(cal_src)
        extra = lambda: cal_dst.copy_(cal_src)  # noqa: E731
    sizes = op_bytes()

    if not names:
        print("bench.py: --ops names none of the suite's ops " + ",".join(ORDER), file=sys.stderr)
        sys.exit(2)
    ms_per_step, per_op = time_ops(torch, ops, names, sizes, args.steps, args.warmup, extra)
    print(f"[bench] suite timed ({args.steps} steps after {args.warmup} warmup)", file=sys.stderr, flush=True)
    ext = None
    if ext_names:
        ext_ms, ext = time_ops(torch, ops, ext_names, sizes, args.steps, args.warmup, None)
        print(f"[bench] extensions timed ({ext_ms:.3f} ms per pass)", file=sys.stderr, flush=True)
    if not args.no_alone:
        time_alone(torch, ops, names, sizes, per_op, args.steps)
        if ext is not None:
            time_alone(torch, ops, ext_names, sizes, ext, args.steps)
        print("[bench] each op timed alone", file=sys.stderr, flush=True)
    total_in = sum(sizes[o][0] for o in names)
    dom = max(names, key=lambda o: per_op[o]["ms"])
    achieved = per_op[dom]["hbm_GBps"]
    traffic = load_traffic(dom)
    st.clear()
    torch.cuda.empty_cache()
    cal = None
    if not args.no_calibration:
        cal = calibrate(torch)
        print("[bench] calibration copy/fill/read timed", file=sys.stderr, flush=True)
    result = {
        "metric": "codec GB/s (fp32 in, encode+EF / decode+accum) and % of MI355X HBM peak",
        "value": round(total_in / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "codec_suite: " + ", ".join(names),
            "uniform": f"{C1_N} fp32, bucket {C1_B}, INT8, EF",
            "fp8_rowwise": f"{C2_ROWS}x{C2_DIM} fp32",
            "qsgd": f"{C3_N} fp32, bucket {C3_B}, s=16, EF",
            "sign": f"{C4_N} bf16, bucket {C4_B}, EF; vote M={C4_M}",
            "accumulate": f"M={C5_M} x {C5_N} INT8, bucket {C5_B}, fused INT8 requant",
            "extensions": (f"outside the step: {X_N} fp32, bucket {X_B}, EF: INT2, stochastic INT4, TernGrad, "
                           f"shared-scale INT8 (max statistic + encode) + decode; M={X_M} x {X_AN}, bucket "
                           f"{X_AB}: TernGrad sum, INT2 sum + INT2 requant, shared-scale INT8 integer sum; "
                           f"tensor list of a {T_L}-layer width-{T_D} transformer ({len(tensor_list_sizes())} "
                           f"tensors, {sum(tensor_list_sizes())} fp32), INT8 + EF, bucket {T_B}: one launch, "
                           f"per-tensor launches, decode into the list; top-k {K_K} of every {K_B} + EF on the "
                           f"{X_N} gradient, its decode, and the sparse sum of {X_M} workers x {X_AN}"),
        },
        "hbm_frac_step": round(sum(sizes[o][1] for o in names) / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": dom,
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_source": (None if traffic is None else
                               "cached: rocprofv3 FETCH_SIZE + WRITE_SIZE runs of this kernel source, "
                               "profiles/pmc_traffic_codec_suite.json (dropped when the source changes)"),
        },
        "calibration": cal,
        "ops": per_op,
    }
    if ext is not None:
        result["extensions"] = ext
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result))


if __name__ == "__main__":
    main()
