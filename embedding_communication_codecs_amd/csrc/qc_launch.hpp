// qc_launch.hpp -- internal interface between the C ABI (qc_api.cpp) and
// the kernel sources.  Arguments arrive here already validated: pointers
// non-NULL where required and 16-byte aligned, sizes positive, bucket a
// power of two in [64, 65536], formats and bit widths supported.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qc {

// Grid-stride kernels never launch more blocks than this.
constexpr int64_t kMaxBlocks = int64_t(1) << 20;

inline int log2_exact(int64_t v) {
    int l = 0;
    while ((int64_t(1) << l) < v) ++l;
    return l;
}

hipError_t launch_encode_uniform(const float* x, float* ef, int64_t n, int32_t bucket, int32_t bits,
                                 bool stochastic, uint64_t seed, uint64_t elem_offset, void* codes,
                                 int64_t payload_bytes, float* scale, float* zero, hipStream_t stream);

// A list of tensors read in place as one concatenated input: the device
// table of their pointers, the device copies of the prefix offsets and the
// per-segment index built by qc_tensor_index, and the total element count.
struct ListSrc {
    const void* const* xs;
    const int64_t* offsets;
    const int32_t* seg_first;
    int32_t ntensors;
    int64_t n;
};

hipError_t launch_encode_uniform_list(const ListSrc& l, float* ef, int32_t bucket, int32_t bits, bool stochastic,
                                      uint64_t seed, uint64_t elem_offset, void* codes, int64_t payload_bytes,
                                      float* scale, float* zero, hipStream_t stream);

hipError_t launch_encode_ternary_list(const ListSrc& l, float* ef, int32_t bucket, uint64_t seed,
                                      uint64_t elem_offset, uint32_t* words, int64_t payload_bytes, float* scale,
                                      hipStream_t stream);

hipError_t launch_encode_qsgd_list(const ListSrc& l, float* ef, int32_t bucket, uint64_t seed, uint64_t elem_offset,
                                   uint32_t* words, int64_t payload_bytes, float* norm, hipStream_t stream);

hipError_t launch_encode_sign_list(const ListSrc& l, bool bf16, float* ef, int32_t bucket, uint32_t* words,
                                   int64_t payload_bytes, float* scale, hipStream_t stream);

hipError_t launch_bucket_absmax_list(const ListSrc& l, const float* ef, int32_t bucket, float* amax,
                                     hipStream_t stream);

hipError_t launch_encode_int8_shared_list(const ListSrc& l, float* ef, int32_t bucket, const float* amax,
                                          uint8_t* codes, int64_t payload_bytes, float* scale, hipStream_t stream);

hipError_t launch_encode_topk_list(const ListSrc& l, float* ef, int32_t bucket, int32_t k, float* values,
                                   uint32_t* indices, hipStream_t stream);

hipError_t launch_encode_ternary(const float* x, float* ef, int64_t n, int32_t bucket, uint64_t seed,
                                 uint64_t elem_offset, uint32_t* words, int64_t payload_bytes,
                                 float* scale, hipStream_t stream);

hipError_t launch_encode_fp8(const float* x, int64_t rows, int32_t dim, uint8_t* codes,
                             int64_t payload_bytes, float* scale, hipStream_t stream);

hipError_t launch_encode_qsgd(const float* x, float* ef, int64_t n, int32_t bucket, uint64_t seed,
                              uint64_t elem_offset, uint32_t* words, int64_t payload_bytes,
                              float* norm, hipStream_t stream);

hipError_t launch_encode_sign(const void* x, bool bf16, float* ef, int64_t n, int32_t bucket,
                              uint32_t* words, int64_t payload_bytes, float* scale,
                              hipStream_t stream);

hipError_t launch_decode(int32_t fmt, const void* codes, const float* scale, const float* zero,
                         int64_t n, int32_t group, int32_t bits, float* out, hipStream_t stream);

hipError_t launch_decode_multi(int32_t fmt, const void* codes, const float* scale, const float* zero,
                               int64_t n, int32_t group, int32_t bits, float* const* outs,
                               const int64_t* offsets, const int32_t* seg_first, int32_t ntensors,
                               hipStream_t stream);

hipError_t launch_dequant_accumulate(int32_t fmt, const void* codes, const float* scale,
                                     const float* zero, int32_t m, int64_t n, int32_t group,
                                     int32_t bits, int64_t payload_bytes, float* acc,
                                     bool accumulate, void* rq_codes, float* rq_scale,
                                     float* rq_zero, hipStream_t stream);

hipError_t launch_bucket_absmax(const float* x, const float* ef, int64_t n, int32_t bucket, float* amax,
                                hipStream_t stream);

hipError_t launch_absmax_combine(const float* amax, int32_t m, int64_t nb, float* out, hipStream_t stream);

hipError_t launch_encode_int8_shared(const float* x, float* ef, int64_t n, int32_t bucket, const float* amax,
                                     uint8_t* codes, int64_t payload_bytes, float* scale, hipStream_t stream);

hipError_t launch_sum_int8_shared(const uint8_t* codes, int32_t m, int64_t n, int32_t bucket,
                                  int64_t payload_bytes, const float* scale, int32_t* isum, bool accumulate,
                                  float* out, hipStream_t stream);

hipError_t launch_encode_topk(const float* x, float* ef, int64_t n, int32_t bucket, int32_t k, float* values,
                              uint32_t* indices, hipStream_t stream);

hipError_t launch_decode_topk(const float* values, const uint32_t* indices, int64_t n, int32_t bucket, int32_t k,
                              float* out, hipStream_t stream);

hipError_t launch_topk_accumulate(const float* values, const uint32_t* indices, int32_t m, int64_t n,
                                  int32_t bucket, int32_t k, float* acc, bool accumulate, hipStream_t stream);

hipError_t launch_majority_vote(const uint32_t* words, int32_t m, int64_t n, int64_t payload_bytes,
                                uint32_t* out_words, hipStream_t stream);

}  // namespace qc
