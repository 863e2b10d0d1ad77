/*
 * qc_oracle.h -- CPU oracle for the quantized-communication codec.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load this library.
 * The GPU library never links it, includes it or calls it, and it shares
 * no source with the GPU library.
 *
 * Everything here is plain, single-threaded, scalar C on host arrays.
 * Floating point is IEEE-754 binary32 with round-to-nearest-even, built
 * without FMA contraction (gcc -ffp-contract=off) and without fast-math,
 * so each fp32 operation written below is one correctly rounded operation
 * in the order written.
 *
 * Pages cited (titles as printed on the pages):
 *   [QCDT]  "Quantized Communication for Distributed Training"
 *   [GQC]   "Gradient quantization for communication"
 *   [QCD]   "Quantization for Communication" (distributed training)
 *   [GCQC]  "Gradient Compression and Quantised Collectives"
 *
 * Shared conventions (readings of points the pages leave open):
 *   - A bucket is `bucket` consecutive elements; the last one may be short.
 *     nb = ceil(n / bucket).  Each bucket has its own statistics.
 *   - Payloads are byte arrays; their size is qco_payload_bytes(), which is
 *     the code bytes rounded up to 16.  Every payload byte is written;
 *     bytes after the last code are zero.
 *   - Low-bit codes are packed least-significant-bit first: element i of a
 *     4-bit payload is bits 4*(i%8)..4*(i%8)+3 of 32-bit word i/8, of a
 *     2-bit payload bits 2*(i%16)..2*(i%16)+1 of word i/16, and of a 1-bit
 *     payload bit i%32 of word i/32 (words little-endian).
 */
#ifndef QC_ORACLE_H
#define QC_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { QCO_UNIFORM = 0, QCO_FP8_ROWWISE = 1, QCO_QSGD = 2, QCO_SIGN = 3, QCO_TERNARY = 4,
       QCO_INT8_SHARED = 5 };

/* Bytes of one payload of n elements (see conventions above). */
int64_t qco_payload_bytes(int32_t fmt, int64_t n, int32_t bits);

/* Philox4x32-10 block function: ctr[4] and key[2] in, out[4] out. */
void qco_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* OCP E4M3FN: code of an fp32 y with |y| <= 448 (RNE), and code -> fp32. */
uint8_t qco_e4m3_from_f32(float y);
float   qco_e4m3_to_f32(uint8_t c);
/* Array form of qco_e4m3_from_f32 (clamps each value to [-448, 448] first). */
void    qco_e4m3_from_f32_n(const float* y, int64_t n, uint8_t* out);

/* Contiguous pairwise sum of len terms, len padded with +0 to `pow2len`. */
float qco_tree_sum(const float* terms, int64_t len, int64_t pow2len);

/* Uniform affine quantizer (bits 8, 4 or 2) with optional error feedback
 * (ef may be NULL): nearest level, or stochastic rounding keyed by
 * (seed, elem_offset + index) as for QSGD. */
void qco_encode_uniform(const float* x, float* ef, int64_t n, int32_t bucket,
                        int32_t bits, uint8_t* payload, float* scale, float* zero);
void qco_encode_uniform_stochastic(const float* x, float* ef, int64_t n, int32_t bucket,
                                   int32_t bits, uint64_t seed, uint64_t elem_offset,
                                   uint8_t* payload, float* scale, float* zero);
void qco_decode_uniform(const uint8_t* payload, const float* scale, const float* zero,
                        int64_t n, int32_t bucket, int32_t bits, float* out);

/* Rowwise FP8-E4M3 for embedding rows. */
void qco_encode_fp8_rowwise(const float* x, int64_t rows, int32_t dim,
                            uint8_t* payload, float* scale);
void qco_decode_fp8_rowwise(const uint8_t* payload, const float* scale,
                            int64_t rows, int32_t dim, float* out);

/* QSGD with 4-bit sign+level codes and error feedback (ef may be NULL).
 * elem_offset is the global index of x[0]; it must be a multiple of 4. */
void qco_encode_qsgd(const float* x, float* ef, int64_t n, int32_t bucket,
                     uint64_t seed, uint64_t elem_offset,
                     uint8_t* payload, float* norm);
void qco_decode_qsgd(const uint8_t* payload, const float* norm, int64_t n,
                     int32_t bucket, float* out);

/* 1-bit sign with per-bucket mean-|v| scale and error feedback (ef may be
 * NULL).  x_bf16 != 0 means x points at bf16 values (uint16 bit patterns),
 * otherwise at fp32 values. */
void qco_encode_sign(const void* x, int32_t x_bf16, float* ef, int64_t n,
                     int32_t bucket, uint8_t* payload, float* scale);
void qco_decode_sign(const uint8_t* payload, const float* scale, int64_t n,
                     int32_t bucket, float* out);

/* TernGrad: codes {0, +1, -1} (2 bits each) times the bucket's max |v|,
 * nonzero with probability |v| / max|v| (ef may be NULL). */
void qco_encode_ternary(const float* x, float* ef, int64_t n, int32_t bucket,
                        uint64_t seed, uint64_t elem_offset,
                        uint8_t* payload, float* scale);
void qco_decode_ternary(const uint8_t* payload, const float* scale, int64_t n,
                        int32_t bucket, float* out);

/* Shared-scale INT8 ("distributed quantization"): every worker encodes a
 * bucket with the same scale, derived from the largest |v| any worker holds
 * there, so the workers' codes add exactly as integers.
 *   qco_bucket_absmax:   amax[k] = max |x + ef| over bucket k (ef may be NULL).
 *   qco_absmax_combine:  out[k] = max over m arrays amax[w*nb + k].
 *   qco_encode_int8_shared: scale = amax/127, symmetric codes in [-127, 127]
 *                        (one int8 per element), error feedback (ef may be NULL).
 *   qco_sum_int8_shared: isum[i] = (accumulate ? isum[i] : 0) + sum of the m
 *                        workers' codes (exact); out[i] = (float)isum[i] * scale.
 *                        isum or out may be NULL (not both); accumulate needs isum. */
void qco_bucket_absmax(const float* x, const float* ef, int64_t n, int32_t bucket, float* amax);
void qco_absmax_combine(const float* amax, int32_t m, int64_t nb, float* out);
void qco_encode_int8_shared(const float* x, float* ef, int64_t n, int32_t bucket,
                            const float* amax, uint8_t* payload, float* scale);
void qco_decode_int8_shared(const uint8_t* payload, const float* scale, int64_t n,
                            int32_t bucket, float* out);
void qco_sum_int8_shared(const uint8_t* payloads, int32_t m, int64_t n, int32_t bucket,
                         const float* scale, int32_t* isum, int32_t accumulate, float* out);

/* Top-k sparsification with error feedback: per bucket, the k_b = min(k,
 * count) coordinates of largest |v| (ties to the smaller index) are sent as
 * (local index, value) pairs in ascending index order, into slots
 * [b*k, b*k + k_b) of values/indices; slots past k_b hold index 0xFFFFFFFF
 * and value +0.  ef (may be NULL) keeps every unsent coordinate whole.
 *   qco_decode_topk:     out = 0 everywhere, then out[b*bucket + idx] = value.
 *   qco_topk_accumulate: acc = (accumulate ? acc : +0); then for each worker
 *                        in order and each valid pair in slot order,
 *                        acc[b*bucket + idx] = acc[...] + value.  Worker w's
 *                        pairs start at w * nb * k. */
void qco_encode_topk(const float* x, float* ef, int64_t n, int32_t bucket, int32_t k,
                     float* values, uint32_t* indices);
void qco_decode_topk(const float* values, const uint32_t* indices, int64_t n, int32_t bucket,
                     int32_t k, float* out);
void qco_topk_accumulate(const float* values, const uint32_t* indices, int32_t m, int64_t n,
                         int32_t bucket, int32_t k, float* acc, int32_t accumulate);

/* Element i of a payload decoded to fp32, for any format. */
float qco_decode_one(int32_t fmt, const uint8_t* payload, const float* scale,
                     const float* zero, int64_t i, int32_t group, int32_t bits);

/* Receive side: acc = (accumulate ? acc : +0) + DQ_0 + DQ_1 + ... + DQ_{m-1},
 * added in worker order.  Worker w's payload starts at
 * w * qco_payload_bytes(fmt, n, bits), its scales at w * ceil(n/group). */
void qco_dequant_accumulate(int32_t fmt, const uint8_t* payloads, const float* scale,
                            const float* zero, int32_t m, int64_t n, int32_t group,
                            int32_t bits, float* acc, int32_t accumulate);

/* signSGD aggregation: output bit p is 1 iff more than half of the m
 * workers have bit p set.  Worker w's words start at
 * w * qco_payload_bytes(QCO_SIGN, n, 1). */
void qco_majority_vote(const uint8_t* payloads, int32_t m, int64_t n, uint8_t* out);

#ifdef __cplusplus
}
#endif
#endif
