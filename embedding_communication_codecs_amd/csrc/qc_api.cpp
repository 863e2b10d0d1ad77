// qc_api.cpp -- the C ABI of libqc (declared in include/qc.h).
//
// Each entry point validates every argument on the host before touching
// the HIP runtime, so a rejected call enqueues nothing and writes nothing,
// and the validation can be exercised on a machine without a GPU.  Valid
// calls hand over to the launchers in the kernel sources.
#include "qc.h"

#include <hip/hip_runtime.h>

#include "qc_launch.hpp"

namespace {

using qc::log2_exact;

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }
bool misaligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) != 0; }
bool misaligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) != 0; }

bool bad_bucket(int32_t b) {
    return b < QC_MIN_BUCKET || b > QC_MAX_BUCKET || (b & (b - 1)) != 0;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int launched(hipError_t e) { return e == hipSuccess ? QC_OK : QC_ERR_LAUNCH; }

hipStream_t hs(qc_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

// Bucket indices are handled as 32-bit values inside some kernels.
constexpr int64_t kMaxBuckets = (int64_t(1) << 31) - 1;

// Largest concatenation a tensor list may describe: far beyond any device
// memory, and small enough that the prefix sums and the per-segment index
// cannot overflow.
constexpr int64_t kMaxListElems = int64_t(1) << 56;

}  // namespace

extern "C" {

int64_t qc_payload_bytes(int32_t fmt, int64_t n, int32_t group, int32_t bits) {
    (void)group;
    if (n < 0) return -1;
    int64_t code_bytes;
    switch (fmt) {
        case QC_UNIFORM:
            if (bits == 8) code_bytes = n;
            else if (bits == 4) code_bytes = 4 * ceil_div(n, 8);
            else if (bits == 2) code_bytes = 4 * ceil_div(n, 16);
            else return -1;
            break;
        case QC_FP8_ROWWISE: code_bytes = n; break;
        case QC_QSGD: code_bytes = 4 * ceil_div(n, 8); break;
        case QC_SIGN: code_bytes = 4 * ceil_div(n, 32); break;
        case QC_TERNARY: code_bytes = 4 * ceil_div(n, 16); break;
        case QC_INT8_SHARED: code_bytes = n; break;
        default: return -1;
    }
    return ceil_div(code_bytes, 16) * 16;
}

const char* qc_status_str(int32_t status) {
    switch (status) {
        case QC_OK: return "QC_OK";
        case QC_ERR_ARG: return "QC_ERR_ARG: invalid argument";
        case QC_ERR_ALIGN: return "QC_ERR_ALIGN: pointer not 16-byte aligned";
        case QC_ERR_UNSUPPORTED: return "QC_ERR_UNSUPPORTED: unsupported format or parameter";
        case QC_ERR_LAUNCH: return "QC_ERR_LAUNCH: kernel launch failed";
        default: return "unknown qc status";
    }
}

namespace {

int encode_uniform_any(const float* x, float* ef, int64_t n, int32_t bucket, int32_t bits,
                       bool stochastic, uint64_t seed, uint64_t elem_offset, void* codes,
                       float* scale, float* zero, qc_stream_t stream) {
    if (n < 0 || bad_bucket(bucket) || (elem_offset & 3u) != 0) return QC_ERR_ARG;
    if (bits != 8 && bits != 4 && bits != 2) return QC_ERR_UNSUPPORTED;
    if (n == 0) return QC_OK;
    if (!x || !codes || !scale || !zero) return QC_ERR_ARG;
    if (ceil_div(n, bucket) > kMaxBuckets) return QC_ERR_ARG;
    if (misaligned(x) || misaligned(ef) || misaligned(codes) || misaligned(scale) || misaligned(zero))
        return QC_ERR_ALIGN;
    return launched(qc::launch_encode_uniform(x, ef, n, bucket, bits, stochastic, seed, elem_offset,
                                              codes, qc_payload_bytes(QC_UNIFORM, n, bucket, bits),
                                              scale, zero, hs(stream)));
}

}  // namespace

int qc_encode_uniform(const float* x, float* ef, int64_t n, int32_t bucket, int32_t bits,
                      void* codes, float* scale, float* zero, qc_stream_t stream) {
    return encode_uniform_any(x, ef, n, bucket, bits, false, 0, 0, codes, scale, zero, stream);
}

int qc_encode_uniform_stochastic(const float* x, float* ef, int64_t n, int32_t bucket, int32_t bits,
                                 uint64_t seed, uint64_t elem_offset, void* codes, float* scale,
                                 float* zero, qc_stream_t stream) {
    return encode_uniform_any(x, ef, n, bucket, bits, true, seed, elem_offset, codes, scale, zero,
                              stream);
}

int qc_tensor_index(const int64_t* sizes, int32_t ntensors, int64_t* offsets, int32_t* seg_first) {
    if (!sizes || !offsets || !seg_first || ntensors < 1) return QC_ERR_ARG;
    // every size is checked, and the total bounded, before anything is written
    int64_t n = 0;
    for (int32_t t = 0; t < ntensors; ++t) {
        if (sizes[t] < 0 || sizes[t] > kMaxListElems - n) return QC_ERR_ARG;
        n += sizes[t];
    }
    offsets[0] = 0;
    for (int32_t t = 0; t < ntensors; ++t) offsets[t + 1] = offsets[t] + sizes[t];
    const int64_t nseg = (n + (int64_t(1) << QC_INDEX_SHIFT) - 1) >> QC_INDEX_SHIFT;
    int32_t t = 0;
    for (int64_t j = 0; j <= nseg; ++j) {
        int64_t g = j << QC_INDEX_SHIFT;
        if (g > n - 1) g = n - 1;
        if (g < 0) g = 0;
        // last tensor whose first element is at or below g (skips empty ones)
        while (t + 1 < ntensors && offsets[t + 1] <= g) ++t;
        seg_first[j] = t;
    }
    return QC_OK;
}

namespace {

// Checks shared by the *_multi encoders: the list tables (validated as far as
// the host can: pointers present and aligned), the bucket, and n.  Returns
// QC_OK with `l` filled, or the error status.
int check_list(const void* const* xs, const int64_t* offsets, const int32_t* seg_first, int32_t ntensors,
               int64_t n, int32_t bucket, qc::ListSrc& l, int32_t max_bucket = QC_MAX_LIST_BUCKET) {
    if (n < 0 || ntensors < 1 || bad_bucket(bucket)) return QC_ERR_ARG;
    if (bucket > max_bucket) return QC_ERR_UNSUPPORTED;
    if (n == 0) return QC_OK;  // an empty call: the caller returns before using l
    if (!xs || !offsets || !seg_first) return QC_ERR_ARG;
    if (ceil_div(n, bucket) > kMaxBuckets) return QC_ERR_ARG;
    if (misaligned8(xs) || misaligned8(offsets) || misaligned4(seg_first)) return QC_ERR_ALIGN;
    l = qc::ListSrc{xs, offsets, seg_first, ntensors, n};
    return QC_OK;
}

int encode_uniform_list(const float* const* xs, const int64_t* offsets, const int32_t* seg_first,
                        int32_t ntensors, int64_t n, float* ef, int32_t bucket, int32_t bits, bool stochastic,
                        uint64_t seed, uint64_t elem_offset, void* codes, float* scale, float* zero,
                        qc_stream_t stream) {
    qc::ListSrc l;
    int st = check_list(reinterpret_cast<const void* const*>(xs), offsets, seg_first, ntensors, n, bucket, l);
    if (st == QC_OK && (elem_offset & 3u) != 0) st = QC_ERR_ARG;
    if (st == QC_OK && bits != 8 && bits != 4 && bits != 2) st = QC_ERR_UNSUPPORTED;
    if (st != QC_OK || n == 0) return st;
    if (!codes || !scale || !zero) return QC_ERR_ARG;
    if (misaligned(ef) || misaligned(codes) || misaligned(scale) || misaligned(zero)) return QC_ERR_ALIGN;
    return launched(qc::launch_encode_uniform_list(l, ef, bucket, bits, stochastic, seed, elem_offset, codes,
                                                   qc_payload_bytes(QC_UNIFORM, n, bucket, bits), scale, zero,
                                                   hs(stream)));
}

}  // namespace

int qc_encode_uniform_multi(const float* const* xs, const int64_t* offsets, const int32_t* seg_first,
                            int32_t ntensors, int64_t n, float* ef, int32_t bucket, int32_t bits, void* codes,
                            float* scale, float* zero, qc_stream_t stream) {
    return encode_uniform_list(xs, offsets, seg_first, ntensors, n, ef, bucket, bits, false, 0, 0, codes, scale,
                               zero, stream);
}

int qc_encode_uniform_stochastic_multi(const float* const* xs, const int64_t* offsets, const int32_t* seg_first,
                                       int32_t ntensors, int64_t n, float* ef, int32_t bucket, int32_t bits,
                                       uint64_t seed, uint64_t elem_offset, void* codes, float* scale, float* zero,
                                       qc_stream_t stream) {
    return encode_uniform_list(xs, offsets, seg_first, ntensors, n, ef, bucket, bits, true, seed, elem_offset,
                               codes, scale, zero, stream);
}

int qc_encode_qsgd_multi(const float* const* xs, const int64_t* offsets, const int32_t* seg_first,
                         int32_t ntensors, int64_t n, float* ef, int32_t bucket, int32_t levels, uint64_t seed,
                         uint64_t elem_offset, uint32_t* words, float* norm, qc_stream_t stream) {
    qc::ListSrc l;
    int st = check_list(reinterpret_cast<const void* const*>(xs), offsets, seg_first, ntensors, n, bucket, l);
    if (st == QC_OK && (elem_offset & 3u) != 0) st = QC_ERR_ARG;
    if (st == QC_OK && levels != 16) st = QC_ERR_UNSUPPORTED;
    if (st != QC_OK || n == 0) return st;
    if (!words || !norm) return QC_ERR_ARG;
    if (misaligned(ef) || misaligned(words) || misaligned(norm)) return QC_ERR_ALIGN;
    return launched(qc::launch_encode_qsgd_list(l, ef, bucket, seed, elem_offset, words,
                                                qc_payload_bytes(QC_QSGD, n, bucket, 16), norm, hs(stream)));
}

int qc_encode_ternary_multi(const float* const* xs, const int64_t* offsets, const int32_t* seg_first,
                            int32_t ntensors, int64_t n, float* ef, int32_t bucket, uint64_t seed,
                            uint64_t elem_offset, uint32_t* words, float* scale, qc_stream_t stream) {
    qc::ListSrc l;
    int st = check_list(reinterpret_cast<const void* const*>(xs), offsets, seg_first, ntensors, n, bucket, l);
    if (st == QC_OK && (elem_offset & 3u) != 0) st = QC_ERR_ARG;
    if (st != QC_OK || n == 0) return st;
    if (!words || !scale) return QC_ERR_ARG;
    if (misaligned(ef) || misaligned(words) || misaligned(scale)) return QC_ERR_ALIGN;
    return launched(qc::launch_encode_ternary_list(l, ef, bucket, seed, elem_offset, words,
                                                   qc_payload_bytes(QC_TERNARY, n, bucket, 2), scale, hs(stream)));
}

int qc_encode_sign_multi(const void* const* xs, int32_t xtype, const int64_t* offsets, const int32_t* seg_first,
                         int32_t ntensors, int64_t n, float* ef, int32_t bucket, uint32_t* words, float* scale,
                         qc_stream_t stream) {
    qc::ListSrc l;
    int st = check_list(xs, offsets, seg_first, ntensors, n, bucket, l);
    if (st == QC_OK && xtype != QC_F32 && xtype != QC_BF16) st = QC_ERR_ARG;
    if (st != QC_OK || n == 0) return st;
    if (!words || !scale) return QC_ERR_ARG;
    if (misaligned(ef) || misaligned(words) || misaligned(scale)) return QC_ERR_ALIGN;
    return launched(qc::launch_encode_sign_list(l, xtype == QC_BF16, ef, bucket, words,
                                                qc_payload_bytes(QC_SIGN, n, bucket, 1), scale, hs(stream)));
}

int qc_bucket_absmax_multi(const float* const* xs, const int64_t* offsets, const int32_t* seg_first,
                           int32_t ntensors, int64_t n, const float* ef, int32_t bucket, float* amax,
                           qc_stream_t stream) {
    qc::ListSrc l;
    const int st = check_list(reinterpret_cast<const void* const*>(xs), offsets, seg_first, ntensors, n, bucket, l);
    if (st != QC_OK || n == 0) return st;
    if (!amax) return QC_ERR_ARG;
    if (misaligned(ef) || misaligned(amax)) return QC_ERR_ALIGN;
    return launched(qc::launch_bucket_absmax_list(l, ef, bucket, amax, hs(stream)));
}

int qc_encode_int8_shared_multi(const float* const* xs, const int64_t* offsets, const int32_t* seg_first,
                                int32_t ntensors, int64_t n, float* ef, int32_t bucket, const float* amax,
                                uint8_t* codes, float* scale, qc_stream_t stream) {
    qc::ListSrc l;
    const int st = check_list(reinterpret_cast<const void* const*>(xs), offsets, seg_first, ntensors, n, bucket, l);
    if (st != QC_OK || n == 0) return st;
    if (!amax || !codes || !scale) return QC_ERR_ARG;
    if (misaligned(ef) || misaligned(amax) || misaligned(codes) || misaligned(scale)) return QC_ERR_ALIGN;
    return launched(qc::launch_encode_int8_shared_list(l, ef, bucket, amax, codes,
                                                       qc_payload_bytes(QC_INT8_SHARED, n, bucket, 8), scale,
                                                       hs(stream)));
}

int qc_encode_fp8_rowwise(const float* x, int64_t rows, int32_t dim, uint8_t* codes, float* scale,
                          qc_stream_t stream) {
    if (rows < 0) return QC_ERR_ARG;
    if (dim < 4 || dim > QC_MAX_BUCKET || dim % 4 != 0) return QC_ERR_UNSUPPORTED;
    if (rows == 0) return QC_OK;
    if (!x || !codes || !scale) return QC_ERR_ARG;
    if (misaligned(x) || misaligned(codes) || misaligned(scale)) return QC_ERR_ALIGN;
    const int64_t n = rows * (int64_t)dim;
    return launched(qc::launch_encode_fp8(x, rows, dim, codes,
                                          qc_payload_bytes(QC_FP8_ROWWISE, n, dim, 8), scale,
                                          hs(stream)));
}

int qc_encode_qsgd(const float* x, float* ef, int64_t n, int32_t bucket, int32_t levels,
                   uint64_t seed, uint64_t elem_offset, uint32_t* words, float* norm,
                   qc_stream_t stream) {
    if (n < 0 || bad_bucket(bucket) || (elem_offset & 3u) != 0) return QC_ERR_ARG;
    if (levels != 16) return QC_ERR_UNSUPPORTED;
    if (n == 0) return QC_OK;
    if (!x || !words || !norm) return QC_ERR_ARG;
    if (ceil_div(n, bucket) > kMaxBuckets) return QC_ERR_ARG;
    if (misaligned(x) || misaligned(ef) || misaligned(words) || misaligned(norm)) return QC_ERR_ALIGN;
    return launched(qc::launch_encode_qsgd(x, ef, n, bucket, seed, elem_offset, words,
                                           qc_payload_bytes(QC_QSGD, n, bucket, 16), norm,
                                           hs(stream)));
}

int qc_encode_ternary(const float* x, float* ef, int64_t n, int32_t bucket, uint64_t seed,
                      uint64_t elem_offset, uint32_t* words, float* scale, qc_stream_t stream) {
    if (n < 0 || bad_bucket(bucket) || (elem_offset & 3u) != 0) return QC_ERR_ARG;
    if (n == 0) return QC_OK;
    if (!x || !words || !scale) return QC_ERR_ARG;
    if (ceil_div(n, bucket) > kMaxBuckets) return QC_ERR_ARG;
    if (misaligned(x) || misaligned(ef) || misaligned(words) || misaligned(scale)) return QC_ERR_ALIGN;
    return launched(qc::launch_encode_ternary(x, ef, n, bucket, seed, elem_offset, words,
                                              qc_payload_bytes(QC_TERNARY, n, bucket, 2), scale,
                                              hs(stream)));
}

int qc_encode_sign(const void* x, int32_t xtype, float* ef, int64_t n, int32_t bucket,
                   uint32_t* words, float* scale, qc_stream_t stream) {
    if (n < 0 || bad_bucket(bucket) || (xtype != QC_F32 && xtype != QC_BF16)) return QC_ERR_ARG;
    if (n == 0) return QC_OK;
    if (!x || !words || !scale) return QC_ERR_ARG;
    if (ceil_div(n, bucket) > kMaxBuckets) return QC_ERR_ARG;
    if (misaligned(x) || misaligned(ef) || misaligned(words) || misaligned(scale)) return QC_ERR_ALIGN;
    return launched(qc::launch_encode_sign(x, xtype == QC_BF16, ef, n, bucket, words,
                                           qc_payload_bytes(QC_SIGN, n, bucket, 1), scale,
                                           hs(stream)));
}

namespace {

// Format/bits/group checks shared by qc_decode and qc_dequant_accumulate.
int check_format(int32_t fmt, int64_t n, int32_t group, int32_t bits, const float* zero,
                 bool accumulate_path) {
    switch (fmt) {
        case QC_UNIFORM:
            if (bits != 8 && bits != 4 && bits != 2) return QC_ERR_UNSUPPORTED;
            if (bad_bucket(group)) return QC_ERR_ARG;
            if (n > 0 && !zero) return QC_ERR_ARG;
            return QC_OK;
        case QC_FP8_ROWWISE:
            if (bits != 8) return QC_ERR_UNSUPPORTED;
            if (group < 4 || group > QC_MAX_BUCKET || group % 4 != 0) return QC_ERR_UNSUPPORTED;
            if (n % group != 0) return QC_ERR_ARG;
            // the accumulator walks 16-element chunks inside one row
            if (accumulate_path && bad_bucket(group)) return QC_ERR_UNSUPPORTED;
            return QC_OK;
        case QC_QSGD:
            if (bits != 16) return QC_ERR_UNSUPPORTED;
            return bad_bucket(group) ? QC_ERR_ARG : QC_OK;
        case QC_SIGN:
            if (bits != 1) return QC_ERR_UNSUPPORTED;
            return bad_bucket(group) ? QC_ERR_ARG : QC_OK;
        case QC_TERNARY:
            if (bits != 2) return QC_ERR_UNSUPPORTED;
            return bad_bucket(group) ? QC_ERR_ARG : QC_OK;
        case QC_INT8_SHARED:
            // payloads with one shared scale are summed by qc_sum_int8_shared
            if (bits != 8 || accumulate_path) return QC_ERR_UNSUPPORTED;
            return bad_bucket(group) ? QC_ERR_ARG : QC_OK;
        default:
            return QC_ERR_UNSUPPORTED;
    }
}

}  // namespace

int qc_decode(int32_t fmt, const void* codes, const float* scale, const float* zero, int64_t n,
              int32_t group, int32_t bits, float* out, qc_stream_t stream) {
    if (n < 0) return QC_ERR_ARG;
    const int st = check_format(fmt, n, group, bits, zero, false);
    if (st != QC_OK) return st;
    if (n == 0) return QC_OK;
    if (!codes || !scale || !out) return QC_ERR_ARG;
    if (ceil_div(n, group) > kMaxBuckets) return QC_ERR_ARG;
    if (misaligned(codes) || misaligned(scale) || misaligned(zero) || misaligned(out))
        return QC_ERR_ALIGN;
    return launched(qc::launch_decode(fmt, codes, scale, zero, n, group, bits, out, hs(stream)));
}

int qc_decode_multi(int32_t fmt, const void* codes, const float* scale, const float* zero, int64_t n,
                    int32_t group, int32_t bits, float* const* outs, const int64_t* offsets,
                    const int32_t* seg_first, int32_t ntensors, qc_stream_t stream) {
    if (n < 0 || ntensors < 1) return QC_ERR_ARG;
    const int st = check_format(fmt, n, group, bits, zero, false);
    if (st != QC_OK) return st;
    if (n == 0) return QC_OK;
    if (!codes || !scale || !outs || !offsets || !seg_first) return QC_ERR_ARG;
    if (ceil_div(n, group) > kMaxBuckets) return QC_ERR_ARG;
    if (misaligned8(outs) || misaligned8(offsets) || misaligned4(seg_first) || misaligned(codes) ||
        misaligned(scale) || misaligned(zero))
        return QC_ERR_ALIGN;
    return launched(qc::launch_decode_multi(fmt, codes, scale, zero, n, group, bits, outs, offsets, seg_first,
                                            ntensors, hs(stream)));
}

int qc_dequant_accumulate(int32_t fmt, const void* codes, const float* scale, const float* zero,
                          int32_t m, int64_t n, int32_t group, int32_t bits, float* acc,
                          int32_t accumulate, void* rq_codes, float* rq_scale, float* rq_zero,
                          qc_stream_t stream) {
    if (n < 0 || m < 1 || m > QC_MAX_WORKERS) return QC_ERR_ARG;
    const int st = check_format(fmt, n, group, bits, zero, true);
    if (st != QC_OK) return st;
    const int rq_set = (rq_codes != nullptr) + (rq_scale != nullptr) + (rq_zero != nullptr);
    if (rq_set != 0 && rq_set != 3) return QC_ERR_ARG;
    if (rq_set == 3 && fmt != QC_UNIFORM) return QC_ERR_UNSUPPORTED;
    if (n == 0) return QC_OK;
    if (!codes || !scale || !acc) return QC_ERR_ARG;
    if (ceil_div(n, group) > kMaxBuckets) return QC_ERR_ARG;
    if (misaligned(codes) || misaligned(scale) || misaligned(zero) || misaligned(acc) ||
        misaligned(rq_codes) || misaligned(rq_scale) || misaligned(rq_zero))
        return QC_ERR_ALIGN;
    const int64_t pbytes = qc_payload_bytes(fmt, n, group, bits);
    return launched(qc::launch_dequant_accumulate(fmt, codes, scale, zero, m, n, group, bits, pbytes,
                                                  acc, accumulate != 0, rq_codes, rq_scale, rq_zero,
                                                  hs(stream)));
}

int qc_bucket_absmax(const float* x, const float* ef, int64_t n, int32_t bucket, float* amax,
                     qc_stream_t stream) {
    if (n < 0 || bad_bucket(bucket)) return QC_ERR_ARG;
    if (n == 0) return QC_OK;
    if (!x || !amax) return QC_ERR_ARG;
    if (ceil_div(n, bucket) > kMaxBuckets) return QC_ERR_ARG;
    if (misaligned(x) || misaligned(ef) || misaligned(amax)) return QC_ERR_ALIGN;
    return launched(qc::launch_bucket_absmax(x, ef, n, bucket, amax, hs(stream)));
}

int qc_absmax_combine(const float* amax, int32_t m, int64_t nb, float* out, qc_stream_t stream) {
    if (nb < 0 || m < 1 || m > QC_MAX_WORKERS || nb > kMaxBuckets) return QC_ERR_ARG;
    if (nb == 0) return QC_OK;
    if (!amax || !out) return QC_ERR_ARG;
    if (misaligned(amax) || misaligned(out)) return QC_ERR_ALIGN;
    return launched(qc::launch_absmax_combine(amax, m, nb, out, hs(stream)));
}

int qc_encode_int8_shared(const float* x, float* ef, int64_t n, int32_t bucket, const float* amax,
                          uint8_t* codes, float* scale, qc_stream_t stream) {
    if (n < 0 || bad_bucket(bucket)) return QC_ERR_ARG;
    if (n == 0) return QC_OK;
    if (!x || !amax || !codes || !scale) return QC_ERR_ARG;
    if (ceil_div(n, bucket) > kMaxBuckets) return QC_ERR_ARG;
    if (misaligned(x) || misaligned(ef) || misaligned(amax) || misaligned(codes) || misaligned(scale))
        return QC_ERR_ALIGN;
    return launched(qc::launch_encode_int8_shared(x, ef, n, bucket, amax, codes,
                                                  qc_payload_bytes(QC_INT8_SHARED, n, bucket, 8), scale,
                                                  hs(stream)));
}

int qc_sum_int8_shared(const uint8_t* codes, int32_t m, int64_t n, int32_t bucket, const float* scale,
                       int32_t* isum, int32_t accumulate, float* out, qc_stream_t stream) {
    if (n < 0 || m < 1 || m > QC_MAX_WORKERS || bad_bucket(bucket)) return QC_ERR_ARG;
    if (!isum && !out) return QC_ERR_ARG;
    if (accumulate && !isum) return QC_ERR_ARG;
    if (n == 0) return QC_OK;
    if (!codes || (out && !scale)) return QC_ERR_ARG;
    if (ceil_div(n, bucket) > kMaxBuckets) return QC_ERR_ARG;
    if (misaligned(codes) || misaligned(scale) || misaligned(isum) || misaligned(out)) return QC_ERR_ALIGN;
    return launched(qc::launch_sum_int8_shared(codes, m, n, bucket, qc_payload_bytes(QC_INT8_SHARED, n, bucket, 8),
                                               scale, isum, accumulate != 0, out, hs(stream)));
}

namespace {

int check_topk(int64_t n, int32_t bucket, int32_t k) {
    if (n < 0 || bad_bucket(bucket) || k < 1 || k > bucket) return QC_ERR_ARG;
    if (bucket > QC_MAX_TOPK_BUCKET) return QC_ERR_UNSUPPORTED;
    if (ceil_div(n, bucket) * (int64_t)k > (int64_t(1) << 40)) return QC_ERR_ARG;
    return QC_OK;
}

}  // namespace

int qc_encode_topk(const float* x, float* ef, int64_t n, int32_t bucket, int32_t k, float* values,
                   uint32_t* indices, qc_stream_t stream) {
    const int st = check_topk(n, bucket, k);
    if (st != QC_OK) return st;
    if (n == 0) return QC_OK;
    if (!x || !values || !indices) return QC_ERR_ARG;
    if (ceil_div(n, bucket) > kMaxBuckets) return QC_ERR_ARG;
    if (misaligned(x) || misaligned(ef) || misaligned4(values) || misaligned4(indices)) return QC_ERR_ALIGN;
    return launched(qc::launch_encode_topk(x, ef, n, bucket, k, values, indices, hs(stream)));
}

int qc_encode_topk_multi(const float* const* xs, const int64_t* offsets, const int32_t* seg_first,
                         int32_t ntensors, int64_t n, float* ef, int32_t bucket, int32_t k, float* values,
                         uint32_t* indices, qc_stream_t stream) {
    qc::ListSrc l;
    int st = check_topk(n, bucket, k);
    if (st == QC_OK)
        st = check_list(reinterpret_cast<const void* const*>(xs), offsets, seg_first, ntensors, n, bucket, l,
                        QC_MAX_TOPK_BUCKET);
    if (st != QC_OK || n == 0) return st;
    if (!values || !indices) return QC_ERR_ARG;
    if (misaligned(ef) || misaligned4(values) || misaligned4(indices)) return QC_ERR_ALIGN;
    return launched(qc::launch_encode_topk_list(l, ef, bucket, k, values, indices, hs(stream)));
}

int qc_decode_topk(const float* values, const uint32_t* indices, int64_t n, int32_t bucket, int32_t k,
                   float* out, qc_stream_t stream) {
    const int st = check_topk(n, bucket, k);
    if (st != QC_OK) return st;
    if (n == 0) return QC_OK;
    if (!values || !indices || !out) return QC_ERR_ARG;
    if (ceil_div(n, bucket) > kMaxBuckets) return QC_ERR_ARG;
    if (misaligned4(values) || misaligned4(indices) || misaligned(out)) return QC_ERR_ALIGN;
    return launched(qc::launch_decode_topk(values, indices, n, bucket, k, out, hs(stream)));
}

int qc_topk_accumulate(const float* values, const uint32_t* indices, int32_t m, int64_t n, int32_t bucket,
                       int32_t k, float* acc, int32_t accumulate, qc_stream_t stream) {
    if (m < 1 || m > QC_MAX_WORKERS) return QC_ERR_ARG;
    const int st = check_topk(n, bucket, k);
    if (st != QC_OK) return st;
    if (n == 0) return QC_OK;
    if (!values || !indices || !acc) return QC_ERR_ARG;
    if (ceil_div(n, bucket) > kMaxBuckets) return QC_ERR_ARG;
    if (misaligned4(values) || misaligned4(indices) || misaligned(acc)) return QC_ERR_ALIGN;
    return launched(qc::launch_topk_accumulate(values, indices, m, n, bucket, k, acc, accumulate != 0, hs(stream)));
}

int qc_majority_vote(const uint32_t* words, int32_t m, int64_t n, uint32_t* out_words,
                     qc_stream_t stream) {
    if (n < 0 || m < 1 || m > QC_MAX_WORKERS) return QC_ERR_ARG;
    if (n == 0) return QC_OK;
    if (!words || !out_words) return QC_ERR_ARG;
    if (misaligned(words) || misaligned(out_words)) return QC_ERR_ALIGN;
    return launched(qc::launch_majority_vote(words, m, n, qc_payload_bytes(QC_SIGN, n, 64, 1),
                                             out_words, hs(stream)));
}

}  // extern "C"
