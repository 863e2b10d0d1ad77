// k_decode.hip -- payload -> fp32 for every wire format.
//
// Each lane turns a chunk of 4 consecutive elements into one 16-byte store,
// so every store instruction of a wave writes 1 KiB contiguously (decoding
// writes 2-32x more bytes than it reads).  A lane reads the 32-bit code
// word holding its chunk (neighbouring lanes share a word for the sub-byte
// formats; those repeats hit in L1) and the chunk's bucket statistics.
// Each thread handles U chunks per tile, issuing all loads first.
//
// Bounds: the word holding a chunk that starts below n lies inside the
// 16-byte-padded payload, so no read goes past the caller's buffer.
#include "qc_device.hpp"
#include "qc_bucket.hpp"
#include "qc_launch.hpp"

namespace qc {
namespace {

enum { F_U8 = 0, F_U4 = 1, F_FP8 = 2, F_QSGD = 3, F_SIGN = 4, F_U2 = 5, F_TER = 6, F_I8S = 7 };

// The code bits of chunk c (elements 4c..4c+3) in the low bits.
template <int F>
__device__ __forceinline__ uint32_t chunk_word(const uint8_t* __restrict__ codes, int64_t c) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(codes);
    if constexpr (F == F_U8 || F == F_FP8 || F == F_I8S) return w[c];
    else if constexpr (F == F_U4 || F == F_QSGD) return w[c >> 1] >> ((c & 1) * 16);
    else if constexpr (F == F_U2 || F == F_TER) return w[c >> 2] >> ((c & 3) * 8);
    else return w[c >> 3] >> ((c & 7) * 4);
}

// fp32 value of element j (0..3) of a chunk whose code bits are `w`.
template <int F>
__device__ __forceinline__ float chunk_value(uint32_t w, int j, float s, float z) {
    if constexpr (F == F_U8) {
        const float p = (float)((w >> (8 * j)) & 0xFFu) * s;
        return p + z;
    } else if constexpr (F == F_U4) {
        const float p = (float)((w >> (4 * j)) & 0xFu) * s;
        return p + z;
    } else if constexpr (F == F_U2) {
        const float p = (float)((w >> (2 * j)) & 0x3u) * s;
        return p + z;
    } else if constexpr (F == F_TER) {
        const uint32_t code = (w >> (2 * j)) & 0x3u;
        return (code & 1u) ? ((code & 2u) ? -s : s) : 0.0f;
    } else if constexpr (F == F_FP8) {
        return e4m3_decode((w >> (8 * j)) & 0xFFu) * s;
    } else if constexpr (F == F_I8S) {
        return (float)(int32_t)(int8_t)(w >> (8 * j)) * s;
    } else if constexpr (F == F_QSGD) {
        const uint32_t code = (w >> (4 * j)) & 0xFu;
        const uint32_t level = code & 7u;
        const float mag = (float)level * z;  // z carries d = norm/7
        return level == 0u ? 0.0f : ((code & 8u) ? -mag : mag);
    } else {
        return ((w >> j) & 1u) ? -s : s;
    }
}

template <int F, bool POW2, int U, bool FULL>
__device__ __forceinline__ void decode_tile(const uint8_t* __restrict__ codes, const float* __restrict__ scale,
                                            const float* __restrict__ zero, int64_t n, int64_t nchunks,
                                            int64_t group, int gshift, float* __restrict__ out, int64_t t0) {
    uint32_t w[U];
    float s[U], z[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t c = t0 + u * 256 + threadIdx.x;
        w[u] = 0u;
        s[u] = 0.0f;
        z[u] = 0.0f;
        if (FULL || c < nchunks) {
            const int64_t bk = POW2 ? ((c << 2) >> gshift) : ((c << 2) / group);
            w[u] = chunk_word<F>(codes, c);
            s[u] = scale[bk];
            if constexpr (F == F_U8 || F == F_U4 || F == F_U2) z[u] = zero[bk];
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t c = t0 + u * 256 + threadIdx.x;
        if (!FULL && c >= nchunks) continue;
        if constexpr (F == F_QSGD) z[u] = s[u] / 7.0f;
        float o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = chunk_value<F>(w[u], j, s[u], z[u]);
        const int64_t i = c << 2;
        if (FULL || i + 4 <= n) {
            st_f4(out + i, f32x4{o[0], o[1], o[2], o[3]});
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (i + j < n) out[i + j] = o[j];
        }
    }
}

// A tile is 256*U chunks.  Tiles wholly inside n (all but at most the last)
// take the branch-free path, so a thread's U loads issue back to back.
template <int F, bool POW2, int U>
__global__ void __launch_bounds__(256)
k_decode(const uint8_t* __restrict__ codes, const float* __restrict__ scale,
         const float* __restrict__ zero, int64_t n, int64_t group, int gshift, float* __restrict__ out) {
    const int64_t nchunks = (n + 3) >> 2;
    constexpr int64_t TILE = 256 * U;
    for (int64_t t0 = (int64_t)blockIdx.x * TILE; t0 < nchunks; t0 += (int64_t)gridDim.x * TILE) {
        if ((t0 + TILE) * 4 <= n)
            decode_tile<F, POW2, U, true>(codes, scale, zero, n, nchunks, group, gshift, out, t0);
        else
            decode_tile<F, POW2, U, false>(codes, scale, zero, n, nchunks, group, gshift, out, t0);
    }
}

template <int F, bool POW2>
hipError_t launch(const void* codes, const float* scale, const float* zero, int64_t n, int32_t group,
                  float* out, hipStream_t stream) {
    constexpr int U = 4;
    const int64_t nchunks = (n + 3) / 4;
    const dim3 grid((unsigned)grid_for(nchunks, 256 * U)), block(256);
    hipLaunchKernelGGL((k_decode<F, POW2, U>), grid, block, 0, stream, (const uint8_t*)codes, scale,
                       zero, n, (int64_t)group, log2_exact(group), out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(int32_t fmt, const void* codes, const float* scale, const float* zero,
                         int64_t n, int32_t group, int32_t bits, float* out, hipStream_t stream) {
    switch (fmt) {
        case 0:  // uniform
            if (bits == 8) return launch<F_U8, true>(codes, scale, zero, n, group, out, stream);
            if (bits == 4) return launch<F_U4, true>(codes, scale, zero, n, group, out, stream);
            return launch<F_U2, true>(codes, scale, zero, n, group, out, stream);
        case 4:  // ternary
            return launch<F_TER, true>(codes, scale, zero, n, group, out, stream);
        case 5:  // shared-scale int8
            return launch<F_I8S, true>(codes, scale, zero, n, group, out, stream);
        case 1:  // rowwise fp8: group = dim, any multiple of 4
            if ((group & (group - 1)) == 0)
                return launch<F_FP8, true>(codes, scale, zero, n, group, out, stream);
            return launch<F_FP8, false>(codes, scale, zero, n, group, out, stream);
        case 2:
            return launch<F_QSGD, true>(codes, scale, zero, n, group, out, stream);
        default:
            return launch<F_SIGN, true>(codes, scale, zero, n, group, out, stream);
    }
}

}  // namespace qc
