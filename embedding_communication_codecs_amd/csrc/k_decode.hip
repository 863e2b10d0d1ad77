// k_decode.hip -- payload -> fp32 for every wire format.
//
// Each lane turns a chunk of 4 consecutive elements into one 16-byte store,
// so every store instruction of a wave writes 1 KiB contiguously (decoding
// writes 2-32x more bytes than it reads).  A lane reads the 32-bit code
// word holding its chunk (neighbouring lanes share a word for the sub-byte
// formats; those repeats hit in L1) and the chunk's bucket statistics.
// Each thread handles U chunks per tile, issuing all loads first: U = 2
// for a flat output (measured on MI355X: 5-20% faster than U = 4, most for
// the 1-bit decoder; U = 1 and U = 8 are slower), U = 4 for a tensor list,
// whose per-tile table search is then paid half as often.
//
// Bounds: the word holding a chunk that starts below n lies inside the
// 16-byte-padded payload, so no read goes past the caller's buffer.
#include "qc_device.hpp"
#include "qc_bucket.hpp"
#include "qc_launch.hpp"
#include "qc.h"

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

// ------------------------------------------------------------ outputs
// FlatOut: one contiguous array.  TensorOuts: the concatenation of T output
// tensors given by a device table of their pointers and the prefix offsets
// of their sizes (off[0] = 0, off[T] = n): one launch scatters a decoded
// bucket buffer back into a whole list of tensors.  prepare() is called once
// per tile with the tile's element range.

struct FlatOut {
    static constexpr int TILE_CHUNKS = 2;
    float* __restrict__ out;
    __device__ __forceinline__ void prepare(int64_t, int64_t) {}
    template <bool FULL>
    __device__ __forceinline__ void store(int64_t i, int64_t n, const float (&o)[4]) const {
        if (FULL || i + 4 <= n) {
            st_f4(out + i, f32x4{o[0], o[1], o[2], o[3]});
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (i + j < n) out[i + j] = o[j];
        }
    }
};

// Largest t in [lo, hi] with off[t] <= g (off[lo] <= g is required).
__device__ __forceinline__ int32_t tensor_of(const int64_t* __restrict__ off, int32_t lo, int32_t hi, int64_t g) {
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (off[mid] <= g) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// The tensors holding elements [g0, g1): the segment index brackets them
// (two loads), a short binary search tightens the bracket.  Index values are
// clamped to [0, T-1].
__device__ __forceinline__ void tensor_range(const int64_t* __restrict__ off, const int32_t* __restrict__ seg,
                                             int32_t T, int64_t g0, int64_t g1, int32_t& lo, int32_t& hi) {
    int32_t a = seg[g0 >> QC_INDEX_SHIFT], b = seg[((g1 - 1) >> QC_INDEX_SHIFT) + 1];
    a = a < 0 ? 0 : (a > T - 1 ? T - 1 : a);
    b = b < a ? a : (b > T - 1 ? T - 1 : b);
    lo = tensor_of(off, a, b, g0);
    hi = tensor_of(off, lo, b, g1 - 1);
}

struct TensorOuts {
    static constexpr int TILE_CHUNKS = 4;
    float* const* __restrict__ outs;
    const int64_t* __restrict__ off;
    const int32_t* __restrict__ seg;
    int32_t T;
    int32_t lo = 0, hi = 0;
    // A tile inside one tensor (the common case: tensors are usually much
    // larger than a tile) stores through that tensor's pointer without
    // looking anything up per store; the search below costs a few dependent
    // loads of the tables per store.
    float* one = nullptr;  // element g of the tile's only tensor is one[g]
    int64_t one_end = 0;

    __device__ __forceinline__ void prepare(int64_t g0, int64_t g1) {
        tensor_range(off, seg, T, g0, g1, lo, hi);
        one = nullptr;
        if (lo == hi) {
            one_end = off[lo + 1];
            one = outs[lo] - off[lo];
        }
    }

    template <bool FULL>
    __device__ __forceinline__ void store(int64_t i, int64_t n, const float (&o)[4]) const {
        if (one != nullptr && (FULL || i + 4 <= n) && i + 4 <= one_end &&
            (reinterpret_cast<uintptr_t>(one + i) & 15u) == 0) {
            st_f4(one + i, f32x4{o[0], o[1], o[2], o[3]});
            return;
        }
        int32_t t = tensor_of(off, lo, hi, i);
        float* p = outs[t] + (i - off[t]);
        if ((FULL || i + 4 <= n) && i + 4 <= off[t + 1] && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
            st_f4(p, f32x4{o[0], o[1], o[2], o[3]});
            return;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t g = i + j;
            if (!FULL && g >= n) break;
            while (t < hi && g >= off[t + 1]) ++t;
            if (g >= off[t] && g < off[t + 1]) outs[t][g - off[t]] = o[j];
        }
    }
};

// d = fl(a/7) without a division: q0 = fl(a * fl(1/7)), then one correction
// with the exact remainder fma(-7, q0, a).  For every finite a this equals
// the correctly rounded quotient (checked over all 2^32 bit patterns); when
// q0 is a zero, an infinity or NaN it already is the quotient's value (a
// zero q0 means |a/7| is at most half the smallest subnormal, since fl(1/7)
// exceeds 1/7).
__device__ __forceinline__ float div7(float a) {
    constexpr float r7 = 0x1.24924ap-3f;
    const float q0 = a * r7;
    const float q1 = __builtin_fmaf(__builtin_fmaf(-7.0f, q0, a), r7, q0);
    return (q0 == 0.0f || !__builtin_isfinite(q0)) ? q0 : q1;
}

template <int F, bool POW2, int U, bool FULL, class Dst>
__device__ __forceinline__ void decode_tile(const uint8_t* __restrict__ codes, const float* __restrict__ scale,
                                            const float* __restrict__ zero, int64_t n, int64_t nchunks,
                                            int64_t group, int gshift, Dst& dst, int64_t t0) {
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
        if constexpr (F == F_QSGD) z[u] = div7(s[u]);
        float o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = chunk_value<F>(w[u], j, s[u], z[u]);
        dst.template store<FULL>(c << 2, n, o);
    }
}

// A tile is 256*U chunks.  Tiles wholly inside n (all but at most the last)
// take the branch-free path, so a thread's U loads issue back to back.
template <int F, bool POW2, int U, class Dst>
__global__ void __launch_bounds__(256)
k_decode(const uint8_t* __restrict__ codes, const float* __restrict__ scale,
         const float* __restrict__ zero, int64_t n, int64_t group, int gshift, Dst dst) {
    const int64_t nchunks = (n + 3) >> 2;
    constexpr int64_t TILE = 256 * U;
    for (int64_t t0 = (int64_t)blockIdx.x * TILE; t0 < nchunks; t0 += (int64_t)gridDim.x * TILE) {
        const bool full = (t0 + TILE) * 4 <= n;
        dst.prepare(t0 * 4, full ? (t0 + TILE) * 4 : n);
        if (full)
            decode_tile<F, POW2, U, true>(codes, scale, zero, n, nchunks, group, gshift, dst, t0);
        else
            decode_tile<F, POW2, U, false>(codes, scale, zero, n, nchunks, group, gshift, dst, t0);
    }
}

template <int F, bool POW2, class Dst>
hipError_t launch(const void* codes, const float* scale, const float* zero, int64_t n, int32_t group,
                  Dst dst, hipStream_t stream) {
    // a tensor-list output pays a table search per tile: longer tiles there
    constexpr int U = Dst::TILE_CHUNKS;
    const int64_t nchunks = (n + 3) / 4;
    const dim3 grid((unsigned)grid_for(nchunks, 256 * U)), block(256);
    hipLaunchKernelGGL((k_decode<F, POW2, U, Dst>), grid, block, 0, stream, (const uint8_t*)codes, scale,
                       zero, n, (int64_t)group, log2_exact(group), dst);
    return hipGetLastError();
}

template <class Dst>
hipError_t launch_decode_dst(int32_t fmt, const void* codes, const float* scale, const float* zero,
                             int64_t n, int32_t group, int32_t bits, Dst out, hipStream_t stream) {
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

}  // namespace

hipError_t launch_decode(int32_t fmt, const void* codes, const float* scale, const float* zero,
                         int64_t n, int32_t group, int32_t bits, float* out, hipStream_t stream) {
    return launch_decode_dst(fmt, codes, scale, zero, n, group, bits, FlatOut{out}, stream);
}

hipError_t launch_decode_multi(int32_t fmt, const void* codes, const float* scale, const float* zero,
                               int64_t n, int32_t group, int32_t bits, float* const* outs,
                               const int64_t* offsets, const int32_t* seg_first, int32_t ntensors,
                               hipStream_t stream) {
    return launch_decode_dst(fmt, codes, scale, zero, n, group, bits,
                             TensorOuts{outs, offsets, seg_first, ntensors}, stream);
}

}  // namespace qc
