// k_topk.hip -- top-k sparsification with error feedback, its decoder and
// the receive-side sum of several workers' sparse payloads.
//
// Encoder: one block per bucket.  Thread t holds EPT consecutive elements
// of the bucket in registers (v = ef + x).  The k-th largest magnitude key
// (the fp32 bits with the sign cleared, which order like |v|) is found
// exactly by a most-significant-digit radix select: four passes over the
// 31 key bits (8, 8, 8 and 7 bits), each building an LDS histogram of the
// next digit among the elements that match the digits fixed so far.  Then
// every element with a larger key is sent, and of those equal to the
// threshold the ones with the smallest indices, as many as are still
// needed.  One block-wide exclusive scan of (larger, equal) counts gives
// every sent element its slot, so the pairs come out in index order.
//
// Decoder and sum: one block per bucket; the bucket's span of the dense
// output is written with zeros (unless the sum continues from the caller's
// values), then the pairs are placed; a barrier separates workers so the
// additions happen in worker order.
#include "qc_device.hpp"
#include "qc_bucket.hpp"
#include "qc_launch.hpp"

namespace qc {
namespace {

constexpr uint32_t kNoIndex = 0xFFFFFFFFu;

__device__ __forceinline__ uint32_t mag_key(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// Block-wide exclusive scan of two counters (thread order); `lds` holds
// 2 * (T/64) values.  Ends with a barrier, so lds can be reused.
template <int T>
__device__ __forceinline__ void block_exclusive_scan2(uint32_t a, uint32_t b, uint32_t& ea, uint32_t& eb,
                                                      uint32_t* lds) {
    constexpr int NW = T / WAVE;
    uint32_t ia = a, ib = b;  // inclusive scans inside the wave
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
        const uint32_t ta = (uint32_t)__shfl_up((int)ia, off, WAVE);
        const uint32_t tb = (uint32_t)__shfl_up((int)ib, off, WAVE);
        if (lane_id() >= off) {
            ia += ta;
            ib += tb;
        }
    }
    if constexpr (NW > 1) {
        if (lane_id() == WAVE - 1) {
            lds[wave_id()] = ia;
            lds[NW + wave_id()] = ib;
        }
        __syncthreads();
        uint32_t pa = 0, pb = 0;
        for (int w = 0; w < wave_id(); ++w) {
            pa += lds[w];
            pb += lds[NW + w];
        }
        __syncthreads();
        ea = pa + ia - a;
        eb = pb + ib - b;
    } else {
        ea = ia - a;
        eb = ib - b;
    }
}

template <int T, int EPT, bool EF>
__global__ void __launch_bounds__(T)
k_enc_topk(const float* __restrict__ x, float* __restrict__ ef, int64_t n, int64_t nb, int32_t k,
           float* __restrict__ values, uint32_t* __restrict__ indices) {
    constexpr int B = T * EPT;
    __shared__ uint32_t hist[256];
    __shared__ uint32_t bcast[2];
    __shared__ uint32_t scan_lds[2 * (T / WAVE)];

    for (int64_t bk = blockIdx.x; bk < nb; bk += gridDim.x) {
        const int64_t lo = bk * B;
        const int64_t cnt = n - lo < B ? n - lo : B;
        const bool full = cnt == B;
        const uint32_t kb = (uint32_t)((int64_t)k < cnt ? k : cnt);
        const int32_t first = threadIdx.x * EPT;  // local index of this thread's element 0

        float v[EPT];
        if (full && EPT % 4 == 0) {
#pragma unroll
            for (int q = 0; q < EPT / 4; ++q) {
                f32x4 g = ld_stream_f4(x + lo + first + 4 * q);
                if constexpr (EF) g = ld_stream_f4(ef + lo + first + 4 * q) + g;
                v[4 * q] = g.x; v[4 * q + 1] = g.y; v[4 * q + 2] = g.z; v[4 * q + 3] = g.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                float g = 0.0f;
                if (first + e < cnt) {
                    g = x[lo + first + e];
                    if constexpr (EF) g = ef[lo + first + e] + g;
                }
                v[e] = g;
            }
        }

        // threshold key and how many elements equal to it are still needed
        uint32_t thr = 0, need_eq = kb;
        const bool all = kb == (uint32_t)cnt;
        if (!all) {
            uint32_t prefix = 0, pmask = 0, krem = kb;
#pragma unroll 1
            for (int pass = 0; pass < 4; ++pass) {
                const int shift = pass == 3 ? 0 : 23 - 8 * pass;
                const uint32_t dmask = pass == 3 ? 0x7Fu : 0xFFu;
                for (int i = threadIdx.x; i < 256; i += T) hist[i] = 0u;
                __syncthreads();
#pragma unroll
                for (int e = 0; e < EPT; ++e) {
                    const uint32_t key = mag_key(v[e]);
                    if (first + e < cnt && (key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
                }
                __syncthreads();
                if (threadIdx.x < WAVE) {
                    // lane l holds bins 4l..4l+3; suffix sums from the top bin down
                    const int l = lane_id();
                    const uint32_t h0 = hist[4 * l], h1 = hist[4 * l + 1], h2 = hist[4 * l + 2], h3 = hist[4 * l + 3];
                    uint32_t s = h0 + h1 + h2 + h3;
#pragma unroll
                    for (int off = 1; off < WAVE; off <<= 1) {
                        const uint32_t t = (uint32_t)__shfl_down((int)s, off, WAVE);
                        if (l + off < WAVE) s += t;
                    }
                    // s = sum of bins >= 4l; suffix(d) for this lane's bins:
                    const uint32_t s3 = s - h0 - h1 - h2, s2 = s3 + h2, s1 = s2 + h1, s0 = s1 + h0;
                    const uint32_t above = s3 - h3;  // sum of bins >= 4l + 4
                    // the digit d with suffix(d) >= krem > suffix(d + 1)
                    if (s3 >= krem && above < krem) { bcast[0] = 4 * l + 3; bcast[1] = above; }
                    if (s2 >= krem && s3 < krem) { bcast[0] = 4 * l + 2; bcast[1] = s3; }
                    if (s1 >= krem && s2 < krem) { bcast[0] = 4 * l + 1; bcast[1] = s2; }
                    if (s0 >= krem && s1 < krem) { bcast[0] = 4 * l; bcast[1] = s1; }
                }
                __syncthreads();
                const uint32_t d = bcast[0];
                krem -= bcast[1];
                prefix |= d << shift;
                pmask |= dmask << shift;
                __syncthreads();  // bcast is rewritten in the next pass
            }
            thr = prefix;
            need_eq = krem;
        }

        // counts of larger and equal keys in this thread, scanned over the block
        uint32_t gt = 0, eq = 0;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const uint32_t key = mag_key(v[e]);
            if (first + e < cnt) {
                gt += (!all && key > thr) ? 1u : 0u;
                eq += (all || key == thr) ? 1u : 0u;
            }
        }
        uint32_t gt_r, eq_r;
        block_exclusive_scan2<T>(gt, eq, gt_r, eq_r, scan_lds);

        float e_out[EPT];
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const uint32_t key = mag_key(v[e]);
            bool sel = false;
            uint32_t pos = 0;
            if (first + e < cnt) {
                if (!all && key > thr) {
                    sel = true;
                    pos = gt_r + (eq_r < need_eq ? eq_r : need_eq);
                    ++gt_r;
                } else if (all || key == thr) {
                    if (eq_r < need_eq) {
                        sel = true;
                        pos = gt_r + eq_r;
                    }
                    ++eq_r;
                }
            }
            if (sel) {
                values[bk * k + pos] = v[e];
                indices[bk * k + pos] = (uint32_t)(first + e);
            }
            e_out[e] = sel ? v[e] - v[e] : v[e];
        }
        for (int64_t j = (int64_t)kb + threadIdx.x; j < k; j += T) {
            values[bk * k + j] = 0.0f;
            indices[bk * k + j] = kNoIndex;
        }
        if constexpr (EF) {
            if (full && EPT % 4 == 0) {
#pragma unroll
                for (int q = 0; q < EPT / 4; ++q)
                    st_f4(ef + lo + first + 4 * q, f32x4{e_out[4 * q], e_out[4 * q + 1], e_out[4 * q + 2], e_out[4 * q + 3]});
            } else {
#pragma unroll
                for (int e = 0; e < EPT; ++e)
                    if (first + e < cnt) ef[lo + first + e] = e_out[e];
            }
        }
        __syncthreads();  // hist and scan space are reused by the next bucket
    }
}

constexpr int TD = 256;  // threads of the decode and sum kernels

// Zeros over [lo, lo + cnt) of a 16-byte aligned bucket span.
__device__ __forceinline__ void zero_span(float* __restrict__ out, int64_t lo, int64_t cnt) {
    const int64_t q4 = cnt >> 2;
    for (int64_t q = threadIdx.x; q < q4; q += TD) st_f4(out + lo + 4 * q, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
    for (int64_t i = 4 * q4 + threadIdx.x; i < cnt; i += TD) out[lo + i] = 0.0f;
}

__global__ void __launch_bounds__(TD)
k_decode_topk(const float* __restrict__ values, const uint32_t* __restrict__ indices, int64_t n, int64_t nb,
              int32_t bucket, int32_t k, float* __restrict__ out) {
    for (int64_t bk = blockIdx.x; bk < nb; bk += gridDim.x) {
        const int64_t lo = bk * bucket;
        const int64_t cnt = n - lo < bucket ? n - lo : bucket;
        zero_span(out, lo, cnt);
        __syncthreads();  // the zeros are in memory before any value lands
        for (int64_t j = threadIdx.x; j < k; j += TD) {
            const uint32_t idx = indices[bk * k + j];
            if ((int64_t)idx < cnt) out[lo + idx] = values[bk * k + j];
        }
        __syncthreads();
    }
}

// Pairs of one worker within a bucket must have distinct indices (as the
// encoder writes them): within a worker the additions run in parallel.
__global__ void __launch_bounds__(TD)
k_topk_accumulate(const float* __restrict__ values, const uint32_t* __restrict__ indices, int32_t m, int64_t n,
                  int64_t nb, int32_t bucket, int32_t k, float* __restrict__ acc, int32_t accumulate) {
    for (int64_t bk = blockIdx.x; bk < nb; bk += gridDim.x) {
        const int64_t lo = bk * bucket;
        const int64_t cnt = n - lo < bucket ? n - lo : bucket;
        if (!accumulate) zero_span(acc, lo, cnt);
        __syncthreads();
        for (int32_t w = 0; w < m; ++w) {
            const int64_t base = ((int64_t)w * nb + bk) * k;
            for (int64_t j = threadIdx.x; j < k; j += TD) {
                const uint32_t idx = indices[base + j];
                if ((int64_t)idx < cnt) acc[lo + idx] = acc[lo + idx] + values[base + j];
            }
            __syncthreads();  // worker w's additions land before worker w + 1's
        }
    }
}

template <int T, int EPT>
hipError_t launch_enc(const float* x, float* ef, int64_t n, int64_t nb, int32_t k, float* values,
                      uint32_t* indices, hipStream_t stream) {
    const dim3 grid((unsigned)grid_for(nb, 1)), block(T);
    if (ef)
        hipLaunchKernelGGL((k_enc_topk<T, EPT, true>), grid, block, 0, stream, x, ef, n, nb, k, values, indices);
    else
        hipLaunchKernelGGL((k_enc_topk<T, EPT, false>), grid, block, 0, stream, x, ef, n, nb, k, values, indices);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_encode_topk(const float* x, float* ef, int64_t n, int32_t bucket, int32_t k, float* values,
                              uint32_t* indices, hipStream_t stream) {
    const int64_t nb = (n + bucket - 1) / bucket;
    switch (bucket) {
        case 64: return launch_enc<64, 1>(x, ef, n, nb, k, values, indices, stream);
        case 128: return launch_enc<64, 2>(x, ef, n, nb, k, values, indices, stream);
        case 256: return launch_enc<64, 4>(x, ef, n, nb, k, values, indices, stream);
        case 512: return launch_enc<64, 8>(x, ef, n, nb, k, values, indices, stream);
        case 1024: return launch_enc<64, 16>(x, ef, n, nb, k, values, indices, stream);
        case 2048: return launch_enc<128, 16>(x, ef, n, nb, k, values, indices, stream);
        case 4096: return launch_enc<256, 16>(x, ef, n, nb, k, values, indices, stream);
        case 8192: return launch_enc<512, 16>(x, ef, n, nb, k, values, indices, stream);
        case 16384: return launch_enc<1024, 16>(x, ef, n, nb, k, values, indices, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_topk(const float* values, const uint32_t* indices, int64_t n, int32_t bucket, int32_t k,
                              float* out, hipStream_t stream) {
    const int64_t nb = (n + bucket - 1) / bucket;
    hipLaunchKernelGGL(k_decode_topk, dim3((unsigned)grid_for(nb, 1)), dim3(TD), 0, stream, values, indices, n, nb,
                       bucket, k, out);
    return hipGetLastError();
}

hipError_t launch_topk_accumulate(const float* values, const uint32_t* indices, int32_t m, int64_t n,
                                  int32_t bucket, int32_t k, float* acc, bool accumulate, hipStream_t stream) {
    const int64_t nb = (n + bucket - 1) / bucket;
    hipLaunchKernelGGL(k_topk_accumulate, dim3((unsigned)grid_for(nb, 1)), dim3(TD), 0, stream, values, indices, m,
                       n, nb, bucket, k, acc, accumulate ? 1 : 0);
    return hipGetLastError();
}

}  // namespace qc
