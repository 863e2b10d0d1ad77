// k_vote.hip -- signSGD majority vote over m packed sign payloads.
//
// Bit-sliced counting: for each of the 128 bit positions of a 16-byte
// vector, the count of set bits across workers is kept as NLEV bit planes
// c[0..NLEV-1] (c[l] holds bit l of every position's count), updated with a
// ripple of half adders per worker (two logic ops per plane).  The result
// count > m/2 is then evaluated with a bit-sliced comparison against the
// constant T = floor(m/2), from the most significant plane down.  Each
// lane handles one 16-byte vector per iteration, so every load of a wave
// reads 1 KiB contiguously.
#include "qc_device.hpp"
#include "qc_bucket.hpp"
#include "qc_launch.hpp"

namespace qc {
namespace {

template <int NLEV>
__global__ void __launch_bounds__(256)
k_majority_vote(const uint32_t* __restrict__ words, int32_t m, int64_t nvec, int64_t stride_vec,
                int64_t nbits, uint32_t* __restrict__ out) {
    const uint32_t T = (uint32_t)m >> 1;
    for (int64_t vi = (int64_t)blockIdx.x * 256 + threadIdx.x; vi < nvec;
         vi += (int64_t)gridDim.x * 256) {
        u32x4 c[NLEV];
#pragma unroll
        for (int l = 0; l < NLEV; ++l) c[l] = u32x4{0u, 0u, 0u, 0u};
        const uint32_t* p = words + vi * 4;
        int32_t w = 0;
        for (; w + 4 <= m; w += 4) {
            u32x4 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) x[u] = ld_stream_u4(p + (int64_t)(w + u) * stride_vec * 4);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                u32x4 carry = x[u];
#pragma unroll
                for (int l = 0; l < NLEV; ++l) {
                    const u32x4 t = c[l] & carry;
                    c[l] ^= carry;
                    carry = t;
                }
            }
        }
        for (; w < m; ++w) {
            u32x4 carry = ld_stream_u4(p + (int64_t)w * stride_vec * 4);
#pragma unroll
            for (int l = 0; l < NLEV; ++l) {
                const u32x4 t = c[l] & carry;
                c[l] ^= carry;
                carry = t;
            }
        }
        // count > T, most significant plane first
        u32x4 gt = u32x4{0u, 0u, 0u, 0u};
        u32x4 eq = u32x4{~0u, ~0u, ~0u, ~0u};
#pragma unroll
        for (int l = NLEV - 1; l >= 0; --l) {
            if ((T >> l) & 1u) {
                eq &= c[l];
            } else {
                gt |= eq & c[l];
                eq &= ~c[l];
            }
        }
        // zero bits at and past n (padding of the payload)
        uint32_t r[4] = {gt.x, gt.y, gt.z, gt.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t bit0 = (vi * 4 + j) * 32;
            if (bit0 >= nbits) r[j] = 0u;
            else if (bit0 + 32 > nbits) r[j] &= (1u << (nbits - bit0)) - 1u;
        }
        st_u4(out + vi * 4, u32x4{r[0], r[1], r[2], r[3]});
    }
}

template <int NLEV>
hipError_t launch(const uint32_t* words, int32_t m, int64_t n, int64_t pbytes, uint32_t* out,
                  hipStream_t stream) {
    const int64_t nvec = pbytes / 16;
    const dim3 grid((unsigned)grid_for(nvec, 256)), block(256);
    hipLaunchKernelGGL((k_majority_vote<NLEV>), grid, block, 0, stream, words, m, nvec, nvec, n, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_majority_vote(const uint32_t* words, int32_t m, int64_t n, int64_t payload_bytes,
                                uint32_t* out_words, hipStream_t stream) {
    int nlev = 1;
    while ((1 << nlev) <= m) ++nlev;  // planes needed to hold counts 0..m
    switch (nlev) {
#define QC_VOTE(L) case L: return launch<L>(words, m, n, payload_bytes, out_words, stream);
        QC_VOTE(1) QC_VOTE(2) QC_VOTE(3) QC_VOTE(4) QC_VOTE(5) QC_VOTE(6) QC_VOTE(7) QC_VOTE(8)
        QC_VOTE(9) QC_VOTE(10) QC_VOTE(11) QC_VOTE(12) QC_VOTE(13) QC_VOTE(14) QC_VOTE(15) QC_VOTE(16)
#undef QC_VOTE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qc
