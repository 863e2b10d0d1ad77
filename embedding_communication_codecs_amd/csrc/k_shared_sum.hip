// k_shared_sum.hip -- receive side of shared-scale INT8: the m workers'
// codes share one scale per bucket, so they are added as integers (exact,
// in any order) and the sum is dequantized once: out = (float)isum * scale.
// Also the max-combine of the workers' bucket maxima that fixes the scale.
//
// Each lane owns chunks of 16 consecutive elements (one 16-byte load per
// worker); consecutive lanes own consecutive chunks, so every load
// instruction of a wave reads 1 KiB contiguously.  A thread keeps U chunks'
// int32 sums in registers while it walks the workers, with the next UW
// workers' loads in flight.  A 16-element chunk never spans two buckets
// (buckets are powers of two >= 64).
//
// Bounds: a chunk starting below n lies inside the 16-byte-padded payload.
#include "qc_device.hpp"
#include "qc_bucket.hpp"
#include "qc_launch.hpp"

namespace qc {
namespace {

constexpr int U = 2;    // chunks per thread per tile
constexpr int UW = 2;   // workers whose loads are in flight
constexpr int TPB = 256;

__device__ __forceinline__ int32_t sbyte(uint32_t w, int k) { return (int32_t)(int8_t)(w >> (8 * k)); }

template <bool FULL>
__device__ __forceinline__ void load_worker(const uint8_t* __restrict__ codes, int64_t pbytes, int32_t w,
                                            int64_t nchunks, int64_t t0, u32x4 (&c)[U]) {
    const uint8_t* p = codes + (int64_t)w * pbytes;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t ch = t0 + u * TPB + threadIdx.x;
        c[u] = (FULL || ch < nchunks) ? ld_stream_u4(p + ch * 16) : u32x4{0u, 0u, 0u, 0u};
    }
}

template <bool FULL, bool ISUM, bool OUT>
__device__ __forceinline__ void sum_tile(const uint8_t* __restrict__ codes, int32_t m, int64_t n,
                                         int64_t nchunks, int64_t pbytes, int gshift,
                                         const float* __restrict__ scale, int32_t* __restrict__ isum,
                                         int32_t accumulate, float* __restrict__ out, int64_t t0, float* xw) {
    int32_t a[U][16];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t ch = t0 + u * TPB + threadIdx.x;
        const int64_t i = ch * 16;
#pragma unroll
        for (int j = 0; j < 16; ++j) a[u][j] = 0;
        if (ISUM && accumulate && (FULL || ch < nchunks)) {
            if (FULL || i + 16 <= n) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x4 t = ld_stream_u4(isum + i + 4 * q);
                    a[u][4 * q] = (int32_t)t.x; a[u][4 * q + 1] = (int32_t)t.y;
                    a[u][4 * q + 2] = (int32_t)t.z; a[u][4 * q + 3] = (int32_t)t.w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (i + j < n) a[u][j] = isum[i + j];
            }
        }
    }

    // rolling prefetch: slot s holds worker w0 + s; refilled with w0 + s + UW
    // as soon as it has been added (the refill index is clamped, so it needs
    // no branch; loads past the last worker are never added)
    u32x4 slot[UW][U];
#pragma unroll
    for (int s = 0; s < UW; ++s) load_worker<FULL>(codes, pbytes, s < m ? s : m - 1, nchunks, t0, slot[s]);
    for (int32_t w0 = 0; w0 < m; w0 += UW) {
#pragma unroll
        for (int s = 0; s < UW; ++s) {
            if (w0 + s < m) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t wd[4] = {slot[s][u].x, slot[s][u].y, slot[s][u].z, slot[s][u].w};
#pragma unroll
                    for (int j = 0; j < 16; ++j) a[u][j] += sbyte(wd[j >> 2], j & 3);
                }
            }
            const int32_t nxt = w0 + UW + s < m ? w0 + UW + s : m - 1;
            load_worker<FULL>(codes, pbytes, nxt, nchunks, t0, slot[s]);
        }
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t ch = t0 + u * TPB + threadIdx.x;
        if (!FULL && ch >= nchunks) continue;
        const int64_t i = ch * 16;
        const bool whole = FULL || i + 16 <= n;
        if constexpr (ISUM) {
            if (whole) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<u32x4*>(isum + i + 4 * q) =
                        u32x4{(uint32_t)a[u][4 * q], (uint32_t)a[u][4 * q + 1], (uint32_t)a[u][4 * q + 2],
                              (uint32_t)a[u][4 * q + 3]};
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (i + j < n) isum[i + j] = a[u][j];
            }
        }
        if constexpr (OUT) {
            const float sc = scale[i >> gshift];
            float o[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) o[j] = (float)a[u][j] * sc;
            if constexpr (FULL) {
                // the wave's 64 chunks are one 1,024-element span
                store_wave_span16(out + (t0 + u * TPB + wave_id() * WAVE) * 16, o, xw);
            } else if (whole) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<f32x4*>(out + i + 4 * q) = f32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (i + j < n) out[i + j] = o[j];
            }
        }
    }
}

// A tile is TPB*U chunks; tiles wholly inside n take the branch-free path.
template <bool ISUM, bool OUT>
__global__ void __launch_bounds__(TPB)
k_sum_int8_shared(const uint8_t* __restrict__ codes, int32_t m, int64_t n, int64_t pbytes, int gshift,
                  const float* __restrict__ scale, int32_t* __restrict__ isum, int32_t accumulate,
                  float* __restrict__ out) {
    const int64_t nchunks = (n + 15) >> 4;
    constexpr int64_t TILE = (int64_t)TPB * U;
    // one 4 KiB buffer per wave for the output's contiguous stores
    __shared__ __align__(16) float xbuf[TPB / WAVE][1024];
    float* xw = &xbuf[wave_id()][0];
    for (int64_t t0 = (int64_t)blockIdx.x * TILE; t0 < nchunks; t0 += (int64_t)gridDim.x * TILE) {
        if ((t0 + TILE) * 16 <= n)
            sum_tile<true, ISUM, OUT>(codes, m, n, nchunks, pbytes, gshift, scale, isum, accumulate, out, t0, xw);
        else
            sum_tile<false, ISUM, OUT>(codes, m, n, nchunks, pbytes, gshift, scale, isum, accumulate, out, t0, xw);
    }
}

// out[k] = the largest of amax[w*nb + k] over w, taken with the comparison
// "replace when greater" in worker order (so NaN and signed zeros behave
// exactly as that loop does).
__global__ void __launch_bounds__(TPB)
k_absmax_combine(const float* __restrict__ amax, int32_t m, int64_t nb, float* __restrict__ out) {
    for (int64_t k = (int64_t)blockIdx.x * TPB + threadIdx.x; k < nb; k += (int64_t)gridDim.x * TPB) {
        float r = amax[k];
        for (int32_t w = 1; w < m; ++w) {
            const float a = amax[(int64_t)w * nb + k];
            r = a > r ? a : r;
        }
        out[k] = r;
    }
}

}  // namespace

hipError_t launch_sum_int8_shared(const uint8_t* codes, int32_t m, int64_t n, int32_t bucket,
                                  int64_t payload_bytes, const float* scale, int32_t* isum, bool accumulate,
                                  float* out, hipStream_t stream) {
    const int64_t nchunks = (n + 15) / 16;
    const dim3 grid((unsigned)grid_for(nchunks, (int64_t)TPB * U)), block(TPB);
    const int gshift = log2_exact(bucket);
    const int32_t acc = accumulate ? 1 : 0;
    if (isum && out)
        hipLaunchKernelGGL((k_sum_int8_shared<true, true>), grid, block, 0, stream, codes, m, n, payload_bytes,
                           gshift, scale, isum, acc, out);
    else if (isum)
        hipLaunchKernelGGL((k_sum_int8_shared<true, false>), grid, block, 0, stream, codes, m, n, payload_bytes,
                           gshift, scale, isum, acc, out);
    else
        hipLaunchKernelGGL((k_sum_int8_shared<false, true>), grid, block, 0, stream, codes, m, n, payload_bytes,
                           gshift, scale, isum, acc, out);
    return hipGetLastError();
}

hipError_t launch_absmax_combine(const float* amax, int32_t m, int64_t nb, float* out, hipStream_t stream) {
    const dim3 grid((unsigned)grid_for(nb, TPB)), block(TPB);
    hipLaunchKernelGGL(k_absmax_combine, grid, block, 0, stream, amax, m, nb, out);
    return hipGetLastError();
}

}  // namespace qc
