// k_encode.hip -- the flat-buffer uniform encoder entry point (round to nearest and stochastic).
// (the kernels are in k_encode.hpp; the entry points are split over four
// sources so they compile in parallel).
#include "k_encode.hpp"

namespace qc {

hipError_t launch_encode_uniform(const float* x, float* ef, int64_t n, int32_t bucket, int32_t bits,
                                 bool stochastic, uint64_t seed, uint64_t elem_offset, void* codes,
                                 int64_t payload_bytes, float* scale, float* zero, hipStream_t stream) {
    return launch_uniform_src(FlatX{x}, ef, n, bucket, bits, stochastic, seed, elem_offset, codes, payload_bytes,
                              scale, zero, stream);
}

}  // namespace qc
