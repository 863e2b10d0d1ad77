/*
 * qc.h -- C ABI of libqc, the quantized-communication codec for MI355X.
 *
 * The codec wraps a collective: the sender turns a training-precision
 * tensor into a small wire payload before the collective and the receiver
 * turns payloads back into fp32 and aggregates them afterwards
 * ("Quantized Communication for Distributed Training", section "Where
 * Quantization Sits"; "Gradient quantization for communication", section
 * "How Gradient Quantization Works").  This library is the per-GPU part:
 * it never communicates.
 *
 * Common rules for every entry point
 * ----------------------------------
 *  - Array arguments are DEVICE pointers on the current HIP device,
 *    allocated and owned by the caller, 16-byte aligned, and must not
 *    overlap each other (the error-feedback buffer is the one array that is
 *    both read and written).
 *  - Every call validates its arguments on the host first; on any error it
 *    returns the status code with nothing enqueued and nothing written.
 *    Otherwise it only enqueues kernels on `stream` (NULL = the default
 *    stream) and returns QC_OK; results are ready once the stream is
 *    synchronized.  The library allocates no memory and keeps no state
 *    between calls, so calls on different streams are independent.
 *  - n == 0 (or rows == 0) is a valid empty call: QC_OK, nothing enqueued.
 *  - Buckets: `bucket` consecutive elements share one set of statistics.
 *    It must be a power of two in [64, 65536].  The last bucket may be
 *    short; it gets its own statistics.  nb = ceil(n / bucket).
 *  - Payloads: a payload of n codes occupies qc_payload_bytes() bytes
 *    (code bytes rounded up to 16).  Encoders write every byte of it;
 *    bytes after the last code are zero.  4-bit codes are packed eight to a
 *    little-endian 32-bit word, element i in bits 4*(i%8)..4*(i%8)+3 of word
 *    i/8; 2-bit codes sixteen to a word, element i in bits 2*(i%16)..+1 of
 *    word i/16; 1-bit codes thirty-two to a word, element i in bit i%32 of
 *    word i/32.  M payloads of one kind are stored back to back, payload w at
 *    byte offset w * qc_payload_bytes(), its per-bucket fp32 statistics at
 *    element offset w * nb of the scale/zero arrays.
 *  - Arithmetic is IEEE fp32 with round-to-nearest-even, no fused
 *    multiply-add in the codec formulas, correctly rounded division and
 *    square root, and denormals preserved, so results are bit-for-bit
 *    reproducible.  Inputs must be finite.
 */
#ifndef QC_H
#define QC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same underlying type as hipStream_t, so a hipStream_t passes unchanged. */
typedef struct ihipStream_t* qc_stream_t;

enum qc_status {
    QC_OK = 0,
    QC_ERR_ARG = 1,          /* NULL pointer, negative size, bad bucket/m/offset */
    QC_ERR_ALIGN = 2,        /* a device pointer is not 16-byte aligned */
    QC_ERR_UNSUPPORTED = 3,  /* bits/levels/format/dim this entry point lacks */
    QC_ERR_LAUNCH = 4        /* the HIP runtime refused the kernel launch */
};

enum qc_format {
    QC_UNIFORM = 0,
    QC_FP8_ROWWISE = 1,
    QC_QSGD = 2,
    QC_SIGN = 3,
    QC_TERNARY = 4,
    QC_INT8_SHARED = 5
};
enum qc_dtype { QC_F32 = 0, QC_BF16 = 1 };

#define QC_MIN_BUCKET 64
#define QC_MAX_BUCKET 65536
#define QC_MAX_WORKERS 65535

/*
 * Uniform (affine) quantization with optional error feedback.
 * ("Quantization for Communication", section "Quantization Schemes",
 * uniform quantization; section "Error Feedback for Quantization", the
 * implementation steps.)
 *
 * Per bucket, v = ef + x (or v = x when ef is NULL); mn/mx are the bucket's
 * min/max of v (a -0 extreme becomes +0); scale = (mx - mn) / (2^bits - 1);
 * zero = mn; code = rint((v - mn) / scale) clamped to [0, 2^bits - 1]
 * (all codes 0 when scale == 0); DQ = code*scale + zero; and, with ef,
 * ef = v - DQ afterwards.
 *
 *   x      fp32[n], read.
 *   ef     fp32[n], read and written in place, or NULL (no feedback).
 *   bits   8 (one byte per code), 4 (eight codes per word) or 2 (sixteen
 *          codes per word; "Quantization for Communication", section
 *          "Bit-Width Selection", 2-bit).
 *   codes  qc_payload_bytes(QC_UNIFORM, n, bucket, bits) bytes, written.
 *   scale  fp32[nb] written; zero fp32[nb] written.
 * Errors: ARG (NULL x/codes/scale/zero, n < 0, bad bucket), ALIGN,
 *         UNSUPPORTED (bits not 2, 4 or 8).
 */
int qc_encode_uniform(const float* x, float* ef, int64_t n, int32_t bucket, int32_t bits,
                      void* codes, float* scale, float* zero, qc_stream_t stream);

/*
 * Uniform quantization with stochastic rounding ("Quantization for
 * Communication", section "Quantization Schemes", stochastic quantization;
 * "Gradient quantization for communication", section "Quantization
 * Schemes"): the same grid, scale and zero as qc_encode_uniform, but with
 * t = (v - mn) / scale the code is floor(t) + (u < t - floor(t)), capped
 * at 2^bits - 1, so E[DQ] = v.  u is the QSGD draw of element g =
 * elem_offset + index (see qc_encode_qsgd).  Payload format and decoding
 * are those of QC_UNIFORM.
 *
 *   bits, x, ef, codes, scale, zero: as for qc_encode_uniform.
 *   seed, elem_offset: as for qc_encode_qsgd (elem_offset a multiple of 4).
 * Errors: as qc_encode_uniform, plus ARG for elem_offset % 4 != 0.
 */
int qc_encode_uniform_stochastic(const float* x, float* ef, int64_t n, int32_t bucket, int32_t bits,
                                 uint64_t seed, uint64_t elem_offset, void* codes, float* scale,
                                 float* zero, qc_stream_t stream);

/*
 * Bucketing front-end ("Gradient Compression and Quantised Collectives",
 * section "When it breaks").  A model's gradient arrives as hundreds of
 * tensors, many of them tiny; one launch per tensor costs more in launch
 * overhead and short buckets than the codec itself.  This call takes the
 * whole list at once and reads each tensor where it lies, with no copy into
 * a staging buffer first.  Encodes the concatenation of a list
 * of fp32 tensors, in list order, exactly as qc_encode_uniform encodes that
 * concatenation held in one buffer, in one launch and without copying the
 * tensors: buckets run across tensor boundaries; ef, codes, scale and zero
 * are laid out for the concatenation.
 *
 *   xs       device array of ntensors device pointers (tensor t's fp32 data,
 *            any 4-byte alignment).
 *   offsets, seg_first
 *            device copies of the tables qc_tensor_index builds from the
 *            sizes (the bucket plan: built once per list layout).  They
 *            cannot be checked on the host: inconsistent tables give wrong
 *            values (reads stay inside [xs[t], xs[t] + offsets[t+1] -
 *            offsets[t]) and inside the tables).
 *   n        total number of elements (offsets[ntensors]).  Other arguments
 *            as qc_encode_uniform.
 * Errors: ARG (NULL table/outputs, ntensors < 1, n < 0, bad bucket), ALIGN
 *         (xs/offsets not 8-byte aligned, seg_first not 4-byte aligned;
 *         ef/codes/scale/zero not 16-byte aligned), UNSUPPORTED (bits, or
 *         bucket above QC_MAX_LIST_BUCKET).
 */
/*
 * The bucket plan of a tensor list, on the host (no device work): from
 * sizes[t] (elements of tensor t, >= 0) it fills
 *   offsets[0..ntensors]   prefix sums: offsets[0] = 0, offsets[t+1] =
 *                          offsets[t] + sizes[t]; offsets[ntensors] = n;
 *   seg_first[0..nseg]     with nseg = ceil(n / 2^QC_INDEX_SHIFT): the
 *                          tensor holding element min(j << QC_INDEX_SHIFT,
 *                          n - 1), i.e. the last t with offsets[t] at or
 *                          below it (0 when n == 0).
 * The caller copies both to the device for the *_multi calls.
 * Returns QC_OK, or QC_ERR_ARG for NULL arrays, ntensors < 1, a negative
 * size or a total above 2^56 elements; every size is checked before
 * anything is written, so a rejected call leaves offsets and seg_first
 * untouched.
 */
#define QC_INDEX_SHIFT 12
/*
 * Largest bucket the *_multi encoders accept.  At 65,536 the tensor-list
 * kernels need more registers than a lane has and would spill to scratch
 * memory; no kernel of this library uses scratch memory (spilled builds of
 * the flat 65,536-element encoders gave results that differ from their
 * source's), so that one size is left to the flat encoders.
 */
#define QC_MAX_LIST_BUCKET 32768
int qc_tensor_index(const int64_t* sizes, int32_t ntensors, int64_t* offsets, int32_t* seg_first);

int qc_encode_uniform_multi(const float* const* xs, const int64_t* offsets, const int32_t* seg_first,
                            int32_t ntensors, int64_t n, float* ef, int32_t bucket, int32_t bits, void* codes,
                            float* scale, float* zero, qc_stream_t stream);

/*
 * The other encoders over a tensor list, each encoding the concatenation of
 * the list exactly as its flat form (named below) encodes that
 * concatenation held in one buffer, in one launch, reading the tensors in
 * place ("Gradient Compression and Quantised Collectives", section "When it
 * breaks").  xs, offsets, seg_first, ntensors and n are as for
 * qc_encode_uniform_multi; every other argument, the results and the
 * errors are those of the flat form, plus the list errors of
 * qc_encode_uniform_multi (ALIGN for the tables, UNSUPPORTED for buckets
 * above QC_MAX_LIST_BUCKET).  Stochastic codecs draw for global element
 * elem_offset + (index in the concatenation).
 *
 *   qc_encode_uniform_stochastic_multi   qc_encode_uniform_stochastic
 *   qc_encode_qsgd_multi                 qc_encode_qsgd
 *   qc_encode_ternary_multi              qc_encode_ternary
 *   qc_encode_sign_multi                 qc_encode_sign: xs are fp32 or bf16
 *                                        tensors (xtype), any 4- or 2-byte
 *                                        alignment
 *   qc_bucket_absmax_multi               qc_bucket_absmax
 *   qc_encode_int8_shared_multi          qc_encode_int8_shared
 *   qc_encode_topk_multi                 qc_encode_topk: buckets up to
 *                                        QC_MAX_TOPK_BUCKET (65,536; its
 *                                        kernels hold no bucket in
 *                                        registers)
 */
int qc_encode_uniform_stochastic_multi(const float* const* xs, const int64_t* offsets, const int32_t* seg_first,
                                       int32_t ntensors, int64_t n, float* ef, int32_t bucket, int32_t bits,
                                       uint64_t seed, uint64_t elem_offset, void* codes, float* scale, float* zero,
                                       qc_stream_t stream);
int qc_encode_qsgd_multi(const float* const* xs, const int64_t* offsets, const int32_t* seg_first,
                         int32_t ntensors, int64_t n, float* ef, int32_t bucket, int32_t levels, uint64_t seed,
                         uint64_t elem_offset, uint32_t* words, float* norm, qc_stream_t stream);
int qc_encode_ternary_multi(const float* const* xs, const int64_t* offsets, const int32_t* seg_first,
                            int32_t ntensors, int64_t n, float* ef, int32_t bucket, uint64_t seed,
                            uint64_t elem_offset, uint32_t* words, float* scale, qc_stream_t stream);
int qc_encode_sign_multi(const void* const* xs, int32_t xtype, const int64_t* offsets, const int32_t* seg_first,
                         int32_t ntensors, int64_t n, float* ef, int32_t bucket, uint32_t* words, float* scale,
                         qc_stream_t stream);
int qc_bucket_absmax_multi(const float* const* xs, const int64_t* offsets, const int32_t* seg_first,
                           int32_t ntensors, int64_t n, const float* ef, int32_t bucket, float* amax,
                           qc_stream_t stream);
int qc_encode_int8_shared_multi(const float* const* xs, const int64_t* offsets, const int32_t* seg_first,
                                int32_t ntensors, int64_t n, float* ef, int32_t bucket, const float* amax,
                                uint8_t* codes, float* scale, qc_stream_t stream);
int qc_encode_topk_multi(const float* const* xs, const int64_t* offsets, const int32_t* seg_first,
                         int32_t ntensors, int64_t n, float* ef, int32_t bucket, int32_t k, float* values,
                         uint32_t* indices, qc_stream_t stream);

/*
 * Rowwise FP8 (OCP E4M3FN) for embedding-lookup payloads: one byte per
 * value plus one fp32 scale per row ("Quantized Communication for
 * Distributed Training", sections "Numeric Example" and "Pinterest QComms
 * Example").
 *
 * Per row: scale = max|x| / 448; code = E4M3(clamp(x / scale, -448, 448)),
 * rounded to nearest even, sign kept on underflow, never NaN; all codes 0
 * when scale == 0.  DQ = E4M3value(code) * scale.
 *
 *   x      fp32[rows * dim] row-major, read.
 *   dim    elements per row, a multiple of 4 in [4, 65536].
 *   codes  qc_payload_bytes(QC_FP8_ROWWISE, rows*dim, dim, 8) bytes, written.
 *   scale  fp32[rows], written.
 * Errors: ARG (NULL pointer, rows < 0), ALIGN, UNSUPPORTED (dim).
 */
int qc_encode_fp8_rowwise(const float* x, int64_t rows, int32_t dim, uint8_t* codes,
                          float* scale, qc_stream_t stream);

/*
 * QSGD: stochastic quantization to s = 16 codes (4 bits: 32/log2(16) = 8x)
 * with optional error feedback ("Quantization for Communication", sections
 * "Quantized SGD Algorithms" and "Quantization Schemes", stochastic
 * quantization; "Gradient Compression and Quantised Collectives", section
 * "Why sparsification fights the all-reduce", unbiased quantisation).
 *
 * Per bucket, v as above; norm = sqrt(sum of v^2), the sum taken as a
 * contiguous pairwise tree over the bucket (padded with +0); d = norm / 7.
 * A code is a sign bit (bit 3) and a level l in 0..7 (bits 0-2) standing
 * for l*d.  With t = |v| / d, l = floor(t) + (u < t - floor(t)), capped at
 * 7, where u = (r >> 8) * 2^-24 and r is word g%4 of Philox4x32-10 with
 * key (seed low 32 bits, seed high 32 bits) and counter (g/4 low, g/4
 * high, 0, 0), g = elem_offset + element index.  Level 0 gives code 0 and
 * DQ +0; all codes are 0 when d == 0.  With ef: ef = v - DQ.
 *
 *   x, ef       as for qc_encode_uniform.
 *   levels      must be 16.
 *   seed        64-bit generator key; vary it per step.
 *   elem_offset global index of x[0] (for a shard of a larger tensor);
 *               a multiple of 4.
 *   words       qc_payload_bytes(QC_QSGD, n, bucket, 16) bytes, written.
 *   norm        fp32[nb], written (the decoder recomputes d = norm / 7).
 * Errors: ARG (NULL pointer, n < 0, bad bucket, elem_offset % 4 != 0),
 *         ALIGN, UNSUPPORTED (levels != 16).
 */
int qc_encode_qsgd(const float* x, float* ef, int64_t n, int32_t bucket, int32_t levels,
                   uint64_t seed, uint64_t elem_offset, uint32_t* words, float* norm,
                   qc_stream_t stream);

/*
 * TernGrad: three levels {-1, 0, +1} times a per-bucket scale, with
 * optional error feedback ("Quantization for Communication", section
 * "Quantized SGD Algorithms", TernGrad).
 *
 * Per bucket, v as above; s = max |v|.  Element v is sent as sign(v) when
 * u < |v| / s (u the QSGD draw of its global index), else as 0, so
 * E[DQ] = v.  Codes are 2 bits: bit 0 = nonzero, bit 1 = negative (0, 1 =
 * +s, 3 = -s).  All codes are 0 when s == 0.  With ef: ef = v - DQ.
 *
 *   x, ef, seed, elem_offset: as for qc_encode_qsgd.
 *   words  qc_payload_bytes(QC_TERNARY, n, bucket, 2) bytes, written.
 *   scale  fp32[nb] (the per-bucket s), written.
 * Errors: ARG (NULL pointer, n < 0, bad bucket, elem_offset % 4 != 0), ALIGN.
 */
int qc_encode_ternary(const float* x, float* ef, int64_t n, int32_t bucket, uint64_t seed,
                      uint64_t elem_offset, uint32_t* words, float* scale, qc_stream_t stream);

/*
 * 1-bit sign quantization with a per-bucket scale and optional error
 * feedback ("Quantization for Communication", sections "Bit-Width
 * Selection" and "Quantized SGD Algorithms", SignSGD; "Gradient
 * Compression and Quantised Collectives", section "Error feedback is the
 * component that makes it work").
 *
 * Per bucket, v = ef + x (bf16 x widened exactly to fp32); scale = (sum of
 * |v|, contiguous pairwise tree) / (valid elements in the bucket);
 * bit = (v < 0); DQ = bit ? -scale : +scale; with ef: ef = v - DQ.
 *
 *   x      QC_F32: fp32[n]; QC_BF16: bf16[n] (uint16 bit patterns), read.
 *   xtype  QC_F32 or QC_BF16.
 *   ef     fp32[n] or NULL.
 *   words  qc_payload_bytes(QC_SIGN, n, bucket, 1) bytes, written.
 *   scale  fp32[nb], written.
 * Errors: ARG (NULL pointer, n < 0, bad bucket, bad xtype), ALIGN.
 */
int qc_encode_sign(const void* x, int32_t xtype, float* ef, int64_t n, int32_t bucket,
                   uint32_t* words, float* scale, qc_stream_t stream);

/*
 * Decode one payload to fp32 (receive side: "Quantized Communication for
 * Distributed Training", section "Where Quantization Sits").
 *
 *   fmt    QC_UNIFORM: bits 8, 4 or 2, scale and zero per bucket of `group`;
 *          QC_FP8_ROWWISE: group = dim, scale per row, zero unused;
 *          QC_QSGD: bits = 16 (levels), scale = the norm array, zero unused;
 *          QC_SIGN: bits = 1, scale per bucket, zero unused;
 *          QC_TERNARY: bits = 2, scale per bucket, zero unused;
 *          QC_INT8_SHARED: bits = 8, scale per bucket (the shared one), zero
 *          unused (qc_dequant_accumulate rejects it: use qc_sum_int8_shared).
 *   codes  the payload, read.   out  fp32[n], written.
 * DQ is the formula stated for the matching encoder.
 * Errors: ARG (NULL pointer, n < 0, bad group, n % dim != 0 for FP8),
 *         ALIGN, UNSUPPORTED (fmt/bits).
 */
int qc_decode(int32_t fmt, const void* codes, const float* scale, const float* zero, int64_t n,
              int32_t group, int32_t bits, float* out, qc_stream_t stream);

/*
 * qc_decode of a payload whose n elements are the concatenation of a list of
 * tensors (see qc_encode_uniform_multi): element offsets[t] + j is written
 * to outs[t][j].  One launch for the whole list.
 *   outs     device array of ntensors device pointers (fp32, any 4-byte
 *            alignment); offsets and seg_first as for
 *            qc_encode_uniform_multi.
 *   Other arguments as qc_decode.
 * Errors: as qc_decode, plus ARG for NULL outs/offsets/seg_first or
 *         ntensors < 1 and ALIGN for misaligned tables.
 */
int qc_decode_multi(int32_t fmt, const void* codes, const float* scale, const float* zero, int64_t n,
                    int32_t group, int32_t bits, float* const* outs, const int64_t* offsets,
                    const int32_t* seg_first, int32_t ntensors, qc_stream_t stream);

/*
 * Receive-side quantized accumulation in fp32 ("Quantization for
 * Communication", section "Quantization-Aware All-Reduce", quantized
 * accumulation; "Gradient quantization for communication", section "How
 * Gradient Quantization Works": dequantize, then aggregate).
 *
 * acc[i] = (accumulate ? acc[i] : +0) + DQ_0[i] + DQ_1[i] + ... + DQ_{m-1}[i],
 * added in worker order, for m payloads stored back to back (see the
 * common rules).  If rq_codes is non-NULL the summed vector is then
 * requantized with qc_encode_uniform's rule (no error feedback, same
 * bits and bucket = group) into rq_codes/rq_scale/rq_zero, in the same
 * pass (for group = 65,536, by a second kernel that reads the sums back
 * once: the sums of such a group are formed in tiles).
 *
 *   fmt/group/bits as for qc_decode.  m in [1, QC_MAX_WORKERS].
 *   codes   m payloads, read.  scale/zero fp32[m * nb], read.
 *   acc     fp32[n], read if accumulate != 0, written.
 *   rq_*    NULL, or (fmt == QC_UNIFORM only) a payload of
 *           qc_payload_bytes(QC_UNIFORM, n, group, bits) bytes and fp32[nb]
 *           scale and zero arrays, written.
 * Errors: ARG (NULL pointer, bad m/n/group, rq_* partly NULL), ALIGN,
 *         UNSUPPORTED (fmt/bits, requantization of a non-uniform format).
 */
int qc_dequant_accumulate(int32_t fmt, const void* codes, const float* scale, const float* zero,
                          int32_t m, int64_t n, int32_t group, int32_t bits, float* acc,
                          int32_t accumulate, void* rq_codes, float* rq_scale, float* rq_zero,
                          qc_stream_t stream);

/*
 * Shared-scale INT8 ("distributed quantization": "Quantization for
 * Communication", section "Quantization-Aware All-Reduce" -- quantize
 * locally, reduce the quantized data, dequantize after the reduction, with
 * scale and zero point coordinated across processes; section "Practical
 * Considerations" -- mismatched parameters give wrong results; "Gradient
 * Compression and Quantised Collectives", section "Why sparsification
 * fights the all-reduce" -- compressed forms that add directly).
 *
 * The workers agree one scale per bucket before encoding: each computes its
 * per-bucket max |v| (qc_bucket_absmax), the maxima are combined with max
 * over workers (what an all-reduce with max computes; qc_absmax_combine
 * combines m arrays held on one device), and every worker encodes with
 * scale = amax/127 (qc_encode_int8_shared).  Codes are symmetric int8 in
 * [-127, 127] with no zero point, so the workers' codes add exactly as
 * integers in any order, and the receiver dequantizes the sum once
 * (qc_sum_int8_shared).  Payload: one int8 per element, 16-byte padded
 * (qc_payload_bytes(QC_INT8_SHARED, n, bucket, 8)); qc_decode decodes one.
 */

/*
 * amax[k] = max |x[i] + ef[i]| over bucket k (ef may be NULL: max |x[i]|).
 *   x, ef  fp32[n], read.   amax  fp32[nb], written (>= +0).
 * Errors: ARG (NULL x/amax, n < 0, bad bucket), ALIGN.
 */
int qc_bucket_absmax(const float* x, const float* ef, int64_t n, int32_t bucket, float* amax,
                     qc_stream_t stream);

/*
 * out[k] = max over w of amax[w * nb + k] for m arrays of nb values stored
 * back to back, taken in worker order with "replace when greater".
 *   amax  fp32[m * nb], read.   out  fp32[nb], written (may not alias amax).
 * Errors: ARG (NULL pointer, m outside [1, QC_MAX_WORKERS], nb < 0), ALIGN.
 */
int qc_absmax_combine(const float* amax, int32_t m, int64_t nb, float* out, qc_stream_t stream);

/*
 * Encode with the agreed maximum: per bucket k, s = amax[k] / 127; with
 * v = x + ef (or x), code = rint(v / s) clamped to [-127, 127] (0 when
 * s == 0); DQ = code * s; with ef: ef = v - DQ.  scale[k] = s is the same
 * on every worker that used the same amax.
 *   amax   fp32[nb], read (e.g. from qc_absmax_combine).
 *   codes  qc_payload_bytes(QC_INT8_SHARED, n, bucket, 8) bytes, written.
 *   scale  fp32[nb], written.
 * Errors: ARG (NULL x/amax/codes/scale, n < 0, bad bucket), ALIGN.
 */
int qc_encode_int8_shared(const float* x, float* ef, int64_t n, int32_t bucket, const float* amax,
                          uint8_t* codes, float* scale, qc_stream_t stream);

/*
 * Receive side: t[i] = (accumulate ? isum[i] : 0) + c_0[i] + ... + c_{m-1}[i]
 * over m shared-scale payloads stored back to back (payload w at
 * w * qc_payload_bytes(QC_INT8_SHARED, n, bucket, 8)); an exact integer sum.
 * If isum is non-NULL it receives t; if out is non-NULL it receives
 * (float)t[i] * scale[i / bucket] (one rounding).  The caller keeps |t|
 * below 2^31 (127 * workers summed so far).
 *   codes  m payloads, read.   scale  fp32[nb] (the shared scale), read if out.
 *   isum   int32[n], read if accumulate, written; or NULL.
 *   out    fp32[n], written; or NULL.  isum and out may not both be NULL.
 * Errors: ARG (NULL codes, isum and out both NULL, accumulate without isum,
 *         out without scale, bad m/n/bucket), ALIGN.
 */
int qc_sum_int8_shared(const uint8_t* codes, int32_t m, int64_t n, int32_t bucket, const float* scale,
                       int32_t* isum, int32_t accumulate, float* out, qc_stream_t stream);

/*
 * Top-k sparsification with error feedback ("Gradient quantization for
 * communication", section "Quantization Schemes": send only the largest K%
 * of the gradient; "Gradient Compression and Quantised Collectives", the
 * opening section -- only the largest-magnitude coordinates -- and section
 * "Why sparsification fights the all-reduce" -- index-value pairs whose sum
 * is not closed, so their exchange is an all-gather; section "Error
 * feedback is the component that makes it work").
 *
 * Per bucket (the last may be short, count elements), k_b = min(k, count)
 * coordinates of largest |v| are sent, v = x + ef; magnitudes compare as
 * the fp32 bit pattern with the sign cleared, and equal magnitudes go to
 * the smaller index.  Bucket b's pairs fill slots [b*k, b*k + k_b) of
 * values (fp32 v) and indices (uint32 index inside the bucket) in ascending
 * index order; slots [b*k + k_b, (b+1)*k) hold index 0xFFFFFFFF and value
 * +0.  With ef: ef = v for unsent coordinates and v - v (= +0) for sent ones.
 *
 *   bucket  a power of two in [64, QC_MAX_TOPK_BUCKET].  k in [1, bucket].
 *   values, indices  nb * k entries each, written (4-byte aligned).
 * Errors: ARG (NULL x/values/indices, n < 0, bad bucket, k outside
 *         [1, bucket]), UNSUPPORTED (bucket > QC_MAX_TOPK_BUCKET), ALIGN.
 */
#define QC_MAX_TOPK_BUCKET 65536
int qc_encode_topk(const float* x, float* ef, int64_t n, int32_t bucket, int32_t k, float* values,
                   uint32_t* indices, qc_stream_t stream);

/*
 * out[i] = 0 for every i < n, then out[b*bucket + idx] = value for each pair
 * whose idx is below the bucket's count (others, such as 0xFFFFFFFF, are
 * skipped).  Pairs of one bucket must have distinct indices.
 * Errors: as qc_encode_topk (out 16-byte aligned).
 */
int qc_decode_topk(const float* values, const uint32_t* indices, int64_t n, int32_t bucket, int32_t k,
                   float* out, qc_stream_t stream);

/*
 * The receive-side sum of m workers' top-k payloads stored back to back
 * (worker w's pairs at w * nb * k): acc = (accumulate ? acc : +0), then for
 * w = 0..m-1 in order, acc[b*bucket + idx] = acc[b*bucket + idx] + value for
 * each valid pair.  Elements no pair touches keep their value.  The pairs of
 * one worker within a bucket must have distinct indices (as the encoder
 * writes them); repeated indices give an unspecified sum.
 * Errors: as qc_encode_topk, plus ARG for m outside [1, QC_MAX_WORKERS].
 */
int qc_topk_accumulate(const float* values, const uint32_t* indices, int32_t m, int64_t n, int32_t bucket,
                       int32_t k, float* acc, int32_t accumulate, qc_stream_t stream);

/*
 * signSGD aggregation by majority vote ("Quantization for Communication",
 * section "Quantized SGD Algorithms", SignSGD; "Gradient Compression and
 * Quantised Collectives", section "Why sparsification fights the
 * all-reduce", one-bit methods).
 *
 * Output bit p is 1 iff more than m/2 of the m sign payloads have bit p
 * set (a tie at even m gives 0, the "+" of sign(0)).
 *
 *   words      m sign payloads of n bits, back to back, read.
 *   out_words  one sign payload, qc_payload_bytes(QC_SIGN, n, 64, 1) bytes,
 *              written (padding zero).
 * Errors: ARG (NULL pointer, n < 0, m outside [1, QC_MAX_WORKERS]), ALIGN.
 */
int qc_majority_vote(const uint32_t* words, int32_t m, int64_t n, uint32_t* out_words,
                     qc_stream_t stream);

/*
 * Bytes of one payload of n elements: the code bytes (n for INT8/FP8 and
 * shared-scale INT8,
 * 4*ceil(n/8) for 4-bit formats, 4*ceil(n/16) for 2-bit formats,
 * 4*ceil(n/32) for sign) rounded up to 16.
 * `group` is accepted for symmetry and does not change the size.  Returns
 * -1 for an unknown format/bits or n < 0.
 */
int64_t qc_payload_bytes(int32_t fmt, int64_t n, int32_t group, int32_t bits);

/* Static string naming a status code. */
const char* qc_status_str(int32_t status);

#ifdef __cplusplus
}
#endif
#endif /* QC_H */
