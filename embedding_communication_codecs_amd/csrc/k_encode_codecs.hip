// k_encode_codecs.hip -- the flat-buffer QSGD, TernGrad, sign and shared-scale entry points.
// (the kernels are in k_encode.hpp; the entry points are split over four
// sources so they compile in parallel).
#include "k_encode.hpp"

namespace qc {

hipError_t launch_encode_ternary(const float* x, float* ef, int64_t n, int32_t bucket, uint64_t seed,
                                 uint64_t elem_offset, uint32_t* words, int64_t payload_bytes,
                                 float* scale, hipStream_t stream) {
    return launch_ternary_src(FlatX{x}, ef, n, bucket, seed, elem_offset, words, payload_bytes, scale, stream);
}

hipError_t launch_encode_qsgd(const float* x, float* ef, int64_t n, int32_t bucket, uint64_t seed,
                              uint64_t elem_offset, uint32_t* words, int64_t payload_bytes,
                              float* norm, hipStream_t stream) {
    return launch_qsgd_src(FlatX{x}, ef, n, bucket, seed, elem_offset, words, payload_bytes, norm, stream);
}

hipError_t launch_encode_sign(const void* x, bool bf16, float* ef, int64_t n, int32_t bucket,
                              uint32_t* words, int64_t payload_bytes, float* scale,
                              hipStream_t stream) {
    if (bf16)
        return launch_sign_src(FlatBF16{static_cast<const uint16_t*>(x)}, ef, n, bucket, words, payload_bytes, scale,
                               stream);
    return launch_sign_src(FlatX{static_cast<const float*>(x)}, ef, n, bucket, words, payload_bytes, scale, stream);
}

hipError_t launch_bucket_absmax(const float* x, const float* ef, int64_t n, int32_t bucket, float* amax,
                                hipStream_t stream) {
    return launch_absmax_src(FlatX{x}, ef, n, bucket, amax, stream);
}

hipError_t launch_encode_int8_shared(const float* x, float* ef, int64_t n, int32_t bucket, const float* amax,
                                     uint8_t* codes, int64_t payload_bytes, float* scale, hipStream_t stream) {
    return launch_int8_shared_src(FlatX{x}, ef, n, bucket, amax, codes, payload_bytes, scale, stream);
}

}  // namespace qc
