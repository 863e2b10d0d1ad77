// k_encode_list_codecs.hip -- the tensor-list QSGD, TernGrad, sign and shared-scale entry points.
// (the kernels are in k_encode.hpp; the entry points are split over four
// sources so they compile in parallel).
#include "k_encode.hpp"

namespace qc {

hipError_t launch_encode_ternary_list(const ListSrc& l, float* ef, int32_t bucket, uint64_t seed,
                                      uint64_t elem_offset, uint32_t* words, int64_t payload_bytes, float* scale,
                                      hipStream_t stream) {
    return launch_ternary_src(list_f32(l), ef, l.n, bucket, seed, elem_offset, words, payload_bytes, scale, stream);
}

hipError_t launch_encode_qsgd_list(const ListSrc& l, float* ef, int32_t bucket, uint64_t seed, uint64_t elem_offset,
                                   uint32_t* words, int64_t payload_bytes, float* norm, hipStream_t stream) {
    return launch_qsgd_src(list_f32(l), ef, l.n, bucket, seed, elem_offset, words, payload_bytes, norm, stream);
}

hipError_t launch_encode_sign_list(const ListSrc& l, bool bf16, float* ef, int32_t bucket, uint32_t* words,
                                   int64_t payload_bytes, float* scale, hipStream_t stream) {
    if (bf16) {
        const TensorList<uint16_t> src{reinterpret_cast<const uint16_t* const*>(l.xs), l.offsets, l.seg_first,
                                       l.ntensors};
        return launch_sign_src(src, ef, l.n, bucket, words, payload_bytes, scale, stream);
    }
    return launch_sign_src(list_f32(l), ef, l.n, bucket, words, payload_bytes, scale, stream);
}

hipError_t launch_bucket_absmax_list(const ListSrc& l, const float* ef, int32_t bucket, float* amax,
                                     hipStream_t stream) {
    return launch_absmax_src(list_f32(l), ef, l.n, bucket, amax, stream);
}

hipError_t launch_encode_int8_shared_list(const ListSrc& l, float* ef, int32_t bucket, const float* amax,
                                          uint8_t* codes, int64_t payload_bytes, float* scale, hipStream_t stream) {
    return launch_int8_shared_src(list_f32(l), ef, l.n, bucket, amax, codes, payload_bytes, scale, stream);
}

}  // namespace qc
