// k_encode.hpp -- gradient encoders with fused error feedback:
//   uniform INT8/INT4/INT2 (round to nearest or stochastic), QSGD (Philox
//   stochastic rounding, 4-bit), TernGrad, 1-bit sign, and the shared-scale
//   INT8 statistic and encoder.
//
// Every encoder makes one HBM pass: a lane group loads its bucket into
// registers (v = ef + x), reduces the bucket statistic across lanes, then
// quantizes, packs and writes codes and the new residual from registers.
// Each encoder reads its input through a source type: one flat array (fp32
// or bf16) or a list of tensors read in place (see TensorList), so a whole
// list of gradients is encoded as their concatenation in one launch.
//
// Register budget: a 1,024-thread block (16 waves) leaves each lane at most
// 128 registers.  Holding a 65,536-element bucket there takes 64 values per
// lane, which does not fit: such kernels spilled to scratch memory, and
// their gfx950 builds gave results that differ from what their source
// computes (run on the CPU, the same source matched the oracle bit for bit
// on the same inputs).  65,536-element buckets therefore take 512-thread
// blocks (256 registers per lane), and a lane holds half of its 128 values
// at a time: the statistic is reduced over both halves, the half still in
// registers is encoded, and the other half is read again (from L2 or the
// last-level cache) and encoded.  No encoder uses scratch memory.
#pragma once

#include "qc_device.hpp"
#include "qc_bucket.hpp"
#include "qc_launch.hpp"
#include "qc.h"

#include <type_traits>

namespace qc {
namespace {

template <int V>
using ic = std::integral_constant<int, V>;

// A part boundary keeps the compiler from carrying work across it: the
// scheduler may not hoist the next part's loads above the current part's
// use (both parts would be in registers again), and the lane's base offset
// is passed through an empty asm statement (no instruction, no memory
// access), so addresses in the next part are derived from it afresh rather
// than kept in registers since the start of the bucket.
__device__ __forceinline__ void part_boundary(int64_t& base) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" : "+v"(base));
}

// Chunks a lane holds in registers at once (see the register budget above):
// all K, or half of them (64 values) in the 512-thread blocks of
// 65,536-element buckets.
template <class G>
constexpr int held_chunks() {
    return (G::THREADS == 512 && G::K * G::E > 64) ? 64 / G::E : G::K;
}

// --------------------------------------------------------------- loading
// Load chunk k (E = 4 fp32 elements at index i) as v = ef + x.  Elements at
// or past n read as 0 and are masked by the caller.  Error feedback is a
// template parameter so that a full bucket's loads are straight-line code
// the compiler can issue back to back (a runtime branch between them makes
// it drain each load before the next).
template <bool FULL, bool EF>
__device__ __forceinline__ void load4(const float* __restrict__ x, const float* __restrict__ ef,
                                      int64_t i, int64_t n, float (&v)[4]) {
    if (FULL || i + 4 <= n) {
        f32x4 g = ld_stream_f4(x + i);
        if constexpr (EF) g = ld_stream_f4(ef + i) + g;
        v[0] = g.x; v[1] = g.y; v[2] = g.z; v[3] = g.w;
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float g = 0.0f;
            if (i + j < n) {
                g = x[i + j];
                if constexpr (EF) g = ef[i + j] + g;
            }
            v[j] = g;
        }
    }
}

// The residual of a chunk of E elements from index i (E = 4 or 8).
template <bool FULL, int E>
__device__ __forceinline__ void store_ef(float* __restrict__ ef, int64_t i, int64_t n, const float (&e)[E]) {
    if (FULL || i + E <= n) {
#pragma unroll
        for (int q = 0; q < E / 4; ++q)
            st_f4(ef + i + 4 * q, f32x4{e[4 * q], e[4 * q + 1], e[4 * q + 2], e[4 * q + 3]});
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j)
            if (i + j < n) ef[i + j] = e[j];
    }
}

// ------------------------------------------------------------- sources
// Where an encoder reads x from.  A source loads chunk i (E elements, E =
// 16 bytes of input: 4 fp32 or 8 bf16) as fp32 values v = ef + x, with
// elements at or past n read as 0.  prepare() is called once per bucket
// with the bucket's element range.

struct FlatX {
    static constexpr int E = 4;
    const float* __restrict__ x;
    __device__ __forceinline__ void prepare(int64_t, int64_t) {}
    template <bool FULL, bool EF>
    __device__ __forceinline__ void load(const float* __restrict__ ef, int64_t i, int64_t n,
                                         float (&v)[4]) const {
        load4<FULL, EF>(x, ef, i, n, v);
    }
};

// bf16 input is widened exactly (bits << 16) before the residual is added.
struct FlatBF16 {
    static constexpr int E = 8;
    const uint16_t* __restrict__ x;
    __device__ __forceinline__ void prepare(int64_t, int64_t) {}
    template <bool FULL, bool EF>
    __device__ __forceinline__ void load(const float* __restrict__ ef, int64_t i, int64_t n,
                                         float (&v)[8]) const {
        if (FULL || i + 8 <= n) {
            const u32x4 w = ld_u4(x + i);
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[2 * h] = bf16_to_f32(ww[h] & 0xFFFFu);
                v[2 * h + 1] = bf16_to_f32(ww[h] >> 16);
            }
            if constexpr (EF) {
                const f32x4 e0 = ld_f4(ef + i), e1 = ld_f4(ef + i + 4);
                const float ee[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = ee[j] + v[j];
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float g = 0.0f;
                if (i + j < n) {
                    g = bf16_to_f32(x[i + j]);
                    if constexpr (EF) g = ef[i + j] + g;
                }
                v[j] = g;
            }
        }
    }
};

// Largest t in [lo, hi] with off[t] <= g (off[lo] <= g is required).  Empty
// tensors (off[t] == off[t+1]) are skipped by construction.
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
// clamped to [0, T-1], so a corrupt index cannot send a read outside the
// tables.
__device__ __forceinline__ void tensor_range(const int64_t* __restrict__ off, const int32_t* __restrict__ seg,
                                             int32_t T, int64_t g0, int64_t g1, int32_t& lo, int32_t& hi) {
    int32_t a = seg[g0 >> QC_INDEX_SHIFT], b = seg[((g1 - 1) >> QC_INDEX_SHIFT) + 1];
    a = a < 0 ? 0 : (a > T - 1 ? T - 1 : a);
    b = b < a ? a : (b > T - 1 ? T - 1 : b);
    lo = tensor_of(off, a, b, g0);
    hi = tensor_of(off, lo, b, g1 - 1);
}

__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(uint16_t x) { return bf16_to_f32(x); }

// The concatenation of T tensors of element type X (fp32 or bf16), given by
// a device table of their pointers and the prefix offsets of their sizes
// (off[0] = 0, off[t+1] = off[t] + size of tensor t, off[T] = n), read in
// place.
template <class X>
struct TensorList {
    static constexpr int E = 16 / (int)sizeof(X);
    const X* const* __restrict__ xs;
    const int64_t* __restrict__ off;
    const int32_t* __restrict__ seg;  // tensor of element j * 2^QC_INDEX_SHIFT (see qc_tensor_index)
    int32_t T;
    int32_t lo = 0, hi = 0;  // tensors that hold the current bucket

    __device__ __forceinline__ void prepare(int64_t g0, int64_t g1) {
        tensor_range(off, seg, T, g0, g1, lo, hi);
    }

    // x[g] of the concatenation, with t a tensor at or before the one
    // holding g; reads nothing outside tensor t's [0, size) range.
    __device__ __forceinline__ float elem(int32_t& t, int64_t g) const {
        while (t < hi && g >= off[t + 1]) ++t;
        const int64_t o = off[t];
        return (g >= o && g < off[t + 1]) ? widen(xs[t][g - o]) : 0.0f;
    }

    template <bool FULL, bool EF>
    __device__ __forceinline__ void load(const float* __restrict__ ef, int64_t i, int64_t n,
                                         float (&v)[E]) const {
        float e[E];
#pragma unroll
        for (int j = 0; j < E; ++j) e[j] = 0.0f;
        if constexpr (EF) {
            if (FULL || i + E <= n) {
#pragma unroll
                for (int q = 0; q < E / 4; ++q) {
                    const f32x4 t = ld_stream_f4(ef + i + 4 * q);
                    e[4 * q] = t.x; e[4 * q + 1] = t.y; e[4 * q + 2] = t.z; e[4 * q + 3] = t.w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < E; ++j)
                    if (i + j < n) e[j] = ef[i + j];
            }
        }
        float x[E];
#pragma unroll
        for (int j = 0; j < E; ++j) x[j] = 0.0f;
        if (FULL || i < n) {
            int32_t t = tensor_of(off, lo, hi, i);
            const int64_t o = off[t];
            const X* p = xs[t] + (i - o);
            if ((FULL || i + E <= n) && i + E <= off[t + 1] && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
                if constexpr (E == 4) {
                    const f32x4 q = ld_stream_f4(reinterpret_cast<const float*>(p));
                    x[0] = q.x; x[1] = q.y; x[2] = q.z; x[3] = q.w;
                } else {
                    const u32x4 w = ld_stream_u4(p);
                    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        x[2 * h] = bf16_to_f32(ww[h] & 0xFFFFu);
                        x[2 * h + 1] = bf16_to_f32(ww[h] >> 16);
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < E; ++j)
                    if (FULL || i + j < n) x[j] = elem(t, i + j);
            }
        }
#pragma unroll
        for (int j = 0; j < E; ++j) v[j] = EF ? e[j] + x[j] : x[j];
    }
};

// Store the codes of a lane's chunk (4 elements from index i) into the
// payload.  8 bits: one 32-bit word per lane; 4 bits: lanes l and l^1 form
// one word; 2 bits: lanes 4j..4j+3 form one word.  The lanes of a word hold
// consecutive chunks, so each word is written by one lane, and only words
// inside the padded payload are written.
template <int BITS>
__device__ __forceinline__ void store_codes4(uint8_t* __restrict__ codes, int64_t i, int64_t pbytes,
                                             const uint32_t (&q)[4]) {
    if constexpr (BITS == 8) {
        const uint32_t word = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
        if (i < pbytes) st_u32(codes + i, word);
    } else if constexpr (BITS == 4) {
        const uint32_t half = q[0] | (q[1] << 4) | (q[2] << 8) | (q[3] << 12);
        const uint32_t other = lane_xor1(half);
        if ((lane_id() & 1) == 0 && i / 2 < pbytes) st_u32(codes + i / 2, half | (other << 16));
    } else {
        const uint32_t byte = q[0] | (q[1] << 2) | (q[2] << 4) | (q[3] << 6);
        const uint32_t word = group_or<4>(byte << (8 * (lane_id() & 3)));
        if ((lane_id() & 3) == 0 && i / 4 < pbytes) st_u32(codes + i / 4, word);
    }
}

// Uniform draws in [0, 1) for the 4 elements of a chunk starting at global
// index g0 (a multiple of 4): the top 24 bits of the Philox4x32-10 block at
// counter (g0/4, 0) with key = seed, times 2^-24 (exact).
__device__ __forceinline__ void chunk_draws(uint64_t g0, uint32_t k0, uint32_t k1, float (&u)[4]) {
    const uint64_t blk = g0 >> 2;
    const u32x4 r = philox4x32_10((uint32_t)blk, (uint32_t)(blk >> 32), 0u, 0u, k0, k1);
    u[0] = (float)(r.x >> 8) * 0x1p-24f;
    u[1] = (float)(r.y >> 8) * 0x1p-24f;
    u[2] = (float)(r.z >> 8) * 0x1p-24f;
    u[3] = (float)(r.w >> 8) * 0x1p-24f;
}

// The chunks [K0, K0 + KH) of a lane's bucket slice into v[0..KH).
template <class G, int K0, int KH, bool FULL, bool EF, class Src>
__device__ __forceinline__ void load_chunks(const Src& src, const float* __restrict__ ef, int64_t base, int64_t n,
                                            float (&v)[KH][Src::E]) {
#pragma unroll
    for (int k = 0; k < KH; ++k)
        src.template load<FULL, EF>(ef, base + (int64_t)(K0 + k) * G::LPB * Src::E, n, v[k]);
}

// f(ic<P>{}) for P = B .. E-1, in order.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(ic<B>{});
        static_for<B + 1, E>(f);
    }
}

// One bucket in parts of KH chunks per lane (see held_chunks): every part
// is loaded and fed to stat(ic<first chunk>), the statistic is finished by
// reduce(), the last part (still in registers) is encoded, then every other
// part is read again and encoded.  encode(ic<first chunk>) may only write
// the residual of its own part, so later re-reads see unchanged inputs.
template <class G, bool FULL, bool EF, int KH, class Src, class Stat, class Reduce, class Encode>
__device__ __forceinline__ void bucket_in_parts(const Src& src, const float* ef, int64_t& base, int64_t n,
                                                float (&v)[KH][Src::E], Stat&& stat, Reduce&& reduce,
                                                Encode&& encode) {
    constexpr int NP = G::K / KH;
    static_for<0, NP>([&](auto p) {
        constexpr int P = decltype(p)::value;
        if constexpr (P > 0) part_boundary(base);
        load_chunks<G, P * KH, KH, FULL, EF>(src, ef, base, n, v);
        stat(ic<P * KH>{});
    });
    reduce();
    encode(ic<(NP - 1) * KH>{});
    static_for<0, NP - 1>([&](auto p) {
        constexpr int P = decltype(p)::value;
        part_boundary(base);
        load_chunks<G, P * KH, KH, FULL, EF>(src, ef, base, n, v);
        encode(ic<P * KH>{});
    });
}

// ============================================================== uniform
// scale = (max - min) / (2^BITS - 1); t = (v - min) / scale; code = rint(t),
// or (STOCH) floor(t) + (u < frac(t)); DQ = code*scale + min; ef = v - DQ.

template <class G, int BITS, bool EF, bool STOCH, bool FULL, class Src>
__device__ __forceinline__ void uniform_bucket(Src src, float* __restrict__ ef,
                                               int64_t n, int64_t bk, uint32_t k0, uint32_t k1,
                                               uint64_t elem_offset, uint8_t* __restrict__ codes,
                                               int64_t pbytes, float* __restrict__ scale,
                                               float* __restrict__ zero, float* lds) {
    constexpr int LPB = G::LPB, KH = held_chunks<G>();
    constexpr uint32_t L = (1u << BITS) - 1u;
    int64_t base = bk * (int64_t)G::B + lane_offset<G>();
    src.prepare(bk * (int64_t)G::B, FULL ? (bk + 1) * (int64_t)G::B : n);

    float v[KH][4];
    float mn = __builtin_inff(), mx = -__builtin_inff(), sc = 0.0f;
    auto minmax = [&](auto k0c) {
        constexpr int C0 = decltype(k0c)::value;
#pragma unroll
        for (int k = 0; k < KH; ++k)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (FULL || base + (int64_t)(C0 + k) * LPB * 4 + j < n) {
                    mn = fminf(mn, v[k][j]);
                    mx = fmaxf(mx, v[k][j]);
                }
    };
    auto reduce = [&]() {
        mn = group_min<LPB>(mn);
        mx = group_max<LPB>(mx);
        if constexpr (G::W > 1) {
            mn = block_min<G::W>(mn, lds);
            mx = block_max<G::W>(mx, lds);
        }
        mn = mn + 0.0f;  // a -0 extreme becomes +0
        mx = mx + 0.0f;
        sc = (mx - mn) / (float)L;
    };
    auto encode = [&](auto k0c) {
        constexpr int C0 = decltype(k0c)::value;
#pragma unroll
        for (int k = 0; k < KH; ++k) {
            const int64_t i = base + (int64_t)(C0 + k) * LPB * 4;
            float u[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if constexpr (STOCH) {
                if (sc != 0.0f && (FULL || i < n)) chunk_draws(elem_offset + (uint64_t)i, k0, k1, u);
            }
            uint32_t q[4];
            float e[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t c = 0;
                if (sc != 0.0f) {
                    const float t = (v[k][j] - mn) / sc;
                    float r;
                    if constexpr (STOCH) {
                        const float fl = floorf(t);
                        const float frac = t - fl;
                        r = fl + (u[j] < frac ? 1.0f : 0.0f);
                    } else {
                        r = __builtin_rintf(t);
                    }
                    c = (uint32_t)fminf(fmaxf(r, 0.0f), (float)L);
                }
                if (!FULL && i + j >= n) c = 0;
                q[j] = c;
                const float p = (float)c * sc;
                const float dq = p + mn;
                e[j] = v[k][j] - dq;
            }
            store_codes4<BITS>(codes, i, pbytes, q);
            if constexpr (EF) store_ef<FULL, 4>(ef, i, n, e);
        }
    };
    bucket_in_parts<G, FULL, EF>(src, ef, base, n, v, minmax, reduce, encode);
    if (bucket_leader<G>()) {
        scale[bk] = sc;
        zero[bk] = mn;
    }
}

template <class G, int BITS, bool EF, bool STOCH, class Src>
__global__ void __launch_bounds__(G::THREADS)
k_enc_uniform(Src src, float* __restrict__ ef, int64_t n, int64_t nb, uint32_t k0, uint32_t k1,
              uint64_t elem_offset, uint8_t* __restrict__ codes, int64_t pbytes, float* __restrict__ scale,
              float* __restrict__ zero) {
    __shared__ float lds[G::W];
    for (int64_t bk = first_bucket<G>(); bk < nb; bk += bucket_stride<G>()) {
        if ((bk + 1) * (int64_t)G::B <= n)
            uniform_bucket<G, BITS, EF, STOCH, true>(src, ef, n, bk, k0, k1, elem_offset, codes, pbytes,
                                                      scale, zero, lds);
        else
            uniform_bucket<G, BITS, EF, STOCH, false>(src, ef, n, bk, k0, k1, elem_offset, codes, pbytes,
                                                       scale, zero, lds);
    }
}

// ================================================================= QSGD
// norm = sqrt(pairwise sum of v^2); d = norm/7; level = floor(|v|/d) + Bernoulli(frac)
// drawn from Philox4x32-10 word g%4 of counter g/4 (g = global index).

template <class G, bool EF, bool FULL, class Src>
__device__ __forceinline__ void qsgd_bucket(Src src, float* __restrict__ ef,
                                            int64_t n, int64_t bk, uint32_t k0, uint32_t k1,
                                            uint64_t elem_offset, uint8_t* __restrict__ words,
                                            int64_t pbytes, float* __restrict__ norm, float* lds) {
    constexpr int K = G::K, LPB = G::LPB, KH = held_chunks<G>();
    int64_t base = bk * (int64_t)G::B + lane_offset<G>();
    src.prepare(bk * (int64_t)G::B, FULL ? (bk + 1) * (int64_t)G::B : n);

    float v[KH][4];
    float s[K];  // chunk k's sum of squares over the lane group: a subtree of the bucket's tree
    float nrm = 0.0f, d = 0.0f, rd = 0.0f;
    bool dok = false;
    auto sums = [&](auto k0c) {
        constexpr int C0 = decltype(k0c)::value;
#pragma unroll
        for (int k = 0; k < KH; ++k) {
            const float a0 = v[k][0] * v[k][0], a1 = v[k][1] * v[k][1];
            const float a2 = v[k][2] * v[k][2], a3 = v[k][3] * v[k][3];
            s[C0 + k] = group_sum<LPB>((a0 + a1) + (a2 + a3));
        }
    };
    auto reduce = [&]() {
        float ss = tree_sum_regs<K>(s);
        if constexpr (G::W > 1) ss = block_tree_sum<G::W>(ss, lds);
        nrm = sqrtf(ss);
        d = nrm / 7.0f;
        dok = quot_divisor_ok(d);
        if (dok) rd = 1.0f / d;
    };
    auto encode = [&](auto k0c) {
        constexpr int C0 = decltype(k0c)::value;
#pragma unroll
        for (int k = 0; k < KH; ++k) {
            const int64_t i = base + (int64_t)(C0 + k) * LPB * 4;
            uint32_t q[4] = {0u, 0u, 0u, 0u};
            float e[4] = {v[k][0], v[k][1], v[k][2], v[k][3]};
            if (d != 0.0f && (FULL || i < n)) {
                float u[4];
                chunk_draws(elem_offset + (uint64_t)i, k0, k1, u);
                // |v| / d through the bucket's reciprocal (quot_n)
                const float ax[4] = {fabsf(v[k][0]), fabsf(v[k][1]), fabsf(v[k][2]), fabsf(v[k][3])};
                float tq[4];
                quot_n<4>(ax, d, rd, dok, tq);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float t = tq[j];
                    const float fl = floorf(t);
                    const float frac = t - fl;
                    uint32_t level = (uint32_t)fl + (u[j] < frac ? 1u : 0u);
                    level = level < 7u ? level : 7u;
                    if (!FULL && i + j >= n) level = 0;
                    if (level != 0u) {
                        const bool neg = v[k][j] < 0.0f;
                        q[j] = (neg ? 8u : 0u) | level;
                        const float mag = (float)level * d;
                        e[j] = v[k][j] - (neg ? -mag : mag);
                    }
                }
            }
            store_codes4<4>(words, i, pbytes, q);
            if constexpr (EF) store_ef<FULL, 4>(ef, i, n, e);
        }
    };
    bucket_in_parts<G, FULL, EF>(src, ef, base, n, v, sums, reduce, encode);
    if (bucket_leader<G>()) norm[bk] = nrm;
}

template <class G, bool EF, class Src>
__global__ void __launch_bounds__(G::THREADS)
k_enc_qsgd(Src src, float* __restrict__ ef, int64_t n, int64_t nb, uint32_t k0,
           uint32_t k1, uint64_t elem_offset, uint8_t* __restrict__ words, int64_t pbytes,
           float* __restrict__ norm) {
    __shared__ float lds[G::W];
    for (int64_t bk = first_bucket<G>(); bk < nb; bk += bucket_stride<G>()) {
        if ((bk + 1) * (int64_t)G::B <= n)
            qsgd_bucket<G, EF, true>(src, ef, n, bk, k0, k1, elem_offset, words, pbytes, norm, lds);
        else
            qsgd_bucket<G, EF, false>(src, ef, n, bk, k0, k1, elem_offset, words, pbytes, norm, lds);
    }
}

// ============================================================= TernGrad
// s = max |v| over the bucket; code = (u < |v|/s) ? (v < 0 ? 3 : 1) : 0
// (bit 0 = nonzero, bit 1 = negative); DQ = 0 or +-s; ef = v - DQ.

template <class G, bool EF, bool FULL, class Src>
__device__ __forceinline__ void ternary_bucket(Src src, float* __restrict__ ef,
                                               int64_t n, int64_t bk, uint32_t k0, uint32_t k1,
                                               uint64_t elem_offset, uint8_t* __restrict__ words,
                                               int64_t pbytes, float* __restrict__ scale, float* lds) {
    constexpr int LPB = G::LPB, KH = held_chunks<G>();
    int64_t base = bk * (int64_t)G::B + lane_offset<G>();
    src.prepare(bk * (int64_t)G::B, FULL ? (bk + 1) * (int64_t)G::B : n);

    float v[KH][4];
    float s = 0.0f;  // masked elements load as 0 and do not change the max
    auto absmax = [&](auto) {
#pragma unroll
        for (int k = 0; k < KH; ++k)
#pragma unroll
            for (int j = 0; j < 4; ++j) s = fmaxf(s, fabsf(v[k][j]));
    };
    auto reduce = [&]() {
        s = group_max<LPB>(s);
        if constexpr (G::W > 1) s = block_max<G::W>(s, lds);
    };
    auto encode = [&](auto k0c) {
        constexpr int C0 = decltype(k0c)::value;
#pragma unroll
        for (int k = 0; k < KH; ++k) {
            const int64_t i = base + (int64_t)(C0 + k) * LPB * 4;
            uint32_t q[4] = {0u, 0u, 0u, 0u};
            float e[4] = {v[k][0], v[k][1], v[k][2], v[k][3]};
            if (s != 0.0f && (FULL || i < n)) {
                float u[4];
                chunk_draws(elem_offset + (uint64_t)i, k0, k1, u);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float p = fabsf(v[k][j]) / s;  // a masked element has p = 0: never sent
                    if (u[j] < p) {
                        const bool neg = v[k][j] < 0.0f;
                        q[j] = neg ? 3u : 1u;
                        e[j] = v[k][j] - (neg ? -s : s);
                    }
                }
            }
            store_codes4<2>(words, i, pbytes, q);
            if constexpr (EF) store_ef<FULL, 4>(ef, i, n, e);
        }
    };
    bucket_in_parts<G, FULL, EF>(src, ef, base, n, v, absmax, reduce, encode);
    if (bucket_leader<G>()) scale[bk] = s;
}

template <class G, bool EF, class Src>
__global__ void __launch_bounds__(G::THREADS)
k_enc_ternary(Src src, float* __restrict__ ef, int64_t n, int64_t nb, uint32_t k0,
              uint32_t k1, uint64_t elem_offset, uint8_t* __restrict__ words, int64_t pbytes,
              float* __restrict__ scale) {
    __shared__ float lds[G::W];
    for (int64_t bk = first_bucket<G>(); bk < nb; bk += bucket_stride<G>()) {
        if ((bk + 1) * (int64_t)G::B <= n)
            ternary_bucket<G, EF, true>(src, ef, n, bk, k0, k1, elem_offset, words, pbytes, scale, lds);
        else
            ternary_bucket<G, EF, false>(src, ef, n, bk, k0, k1, elem_offset, words, pbytes, scale, lds);
    }
}

// ================================================================= sign
// scale = (pairwise sum of |v|) / count; bit = v < 0; DQ = bit ? -scale : scale.
// fp32 input: chunks of 4 elements; bf16 input: chunks of 8 (16 bytes).

template <class G, bool EF, bool FULL, class Src>
__device__ __forceinline__ void sign_bucket(Src src, float* __restrict__ ef,
                                            int64_t n, int64_t bk, int64_t nb,
                                            uint8_t* __restrict__ words, int64_t pbytes,
                                            float* __restrict__ scale, float* lds) {
    constexpr int K = G::K, LPB = G::LPB, E = G::E, KH = held_chunks<G>();
    static_assert(E == Src::E, "source chunk width");
    int64_t base = bk * (int64_t)G::B + lane_offset<G>();
    src.prepare(bk * (int64_t)G::B, FULL ? (bk + 1) * (int64_t)G::B : n);

    // sum of |v|: chunk-local pairwise tree, then lanes, chunks and waves
    float v[KH][E];
    float s[K];
    float sc = 0.0f;
    auto sums = [&](auto k0c) {
        constexpr int C0 = decltype(k0c)::value;
#pragma unroll
        for (int k = 0; k < KH; ++k) {
            float a[E];
#pragma unroll
            for (int j = 0; j < E; ++j) a[j] = fabsf(v[k][j]);  // masked elements are +0
            s[C0 + k] = group_sum<LPB>(tree_sum_regs<E>(a));
        }
    };
    auto reduce = [&]() {
        float S = tree_sum_regs<K>(s);
        if constexpr (G::W > 1) S = block_tree_sum<G::W>(S, lds);
        const int64_t cnt = FULL ? (int64_t)G::B : n - bk * (int64_t)G::B;
        sc = S / (float)cnt;
    };
    constexpr int LPW = 32 / E;  // lanes per 32-bit output word
    auto encode = [&](auto k0c) {
        constexpr int C0 = decltype(k0c)::value;
#pragma unroll
        for (int k = 0; k < KH; ++k) {
            const int64_t i = base + (int64_t)(C0 + k) * LPB * E;
            uint32_t bits = 0;
            float e[E];
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const bool neg = v[k][j] < 0.0f;  // masked elements load as +0: their bits are 0
                bits |= (neg ? 1u : 0u) << j;
                e[j] = v[k][j] - (neg ? -sc : sc);
            }
            const uint32_t word = group_or<LPW>(bits << (E * (lane_id() % LPW)));
            if (lane_id() % LPW == 0 && i / 8 < pbytes) st_u32(words + i / 8, word);
            if constexpr (EF) store_ef<FULL, E>(ef, i, n, e);
        }
    };
    bucket_in_parts<G, FULL, EF>(src, ef, base, n, v, sums, reduce, encode);
    if (bucket_leader<G>()) {
        scale[bk] = sc;
        // 64-element buckets span 8 bytes; the payload is padded to 16, so
        // the last bucket also zeroes any padding words past its own end.
        if (bk == nb - 1)
            for (int64_t b = (bk + 1) * (int64_t)G::B / 8; b < pbytes; b += 4) st_u32(words + b, 0u);
    }
}

template <class G, bool EF, class Src>
__global__ void __launch_bounds__(G::THREADS)
k_enc_sign(Src src, float* __restrict__ ef, int64_t n, int64_t nb,
           uint8_t* __restrict__ words, int64_t pbytes, float* __restrict__ scale) {
    __shared__ float lds[G::W];
    for (int64_t bk = first_bucket<G>(); bk < nb; bk += bucket_stride<G>()) {
        if ((bk + 1) * (int64_t)G::B <= n)
            sign_bucket<G, EF, true>(src, ef, n, bk, nb, words, pbytes, scale, lds);
        else
            sign_bucket<G, EF, false>(src, ef, n, bk, nb, words, pbytes, scale, lds);
    }
}

// ===================================================== shared-scale INT8
// The bucket statistic each worker contributes: amax = max |v|.  After the
// workers' maxima are combined (max over workers), every worker encodes
// with scale = amax/127: code = rint(v/scale) clamped to [-127, 127] as an
// int8 byte (0 when scale is 0); DQ = code*scale; ef = v - DQ.

template <class G, bool EF, bool FULL, class Src>
__device__ __forceinline__ void absmax_bucket(Src src, const float* __restrict__ ef,
                                              int64_t n, int64_t bk, float* __restrict__ amax, float* lds) {
    constexpr int KH = held_chunks<G>();
    int64_t base = bk * (int64_t)G::B + lane_offset<G>();
    src.prepare(bk * (int64_t)G::B, FULL ? (bk + 1) * (int64_t)G::B : n);
    float v[KH][4];
    float m = 0.0f;  // masked elements load as 0 and do not change the max
    static_for<0, G::K / KH>([&](auto p) {
        constexpr int P = decltype(p)::value;
        if constexpr (P > 0) part_boundary(base);
        load_chunks<G, P * KH, KH, FULL, EF>(src, ef, base, n, v);
#pragma unroll
        for (int k = 0; k < KH; ++k)
#pragma unroll
            for (int j = 0; j < 4; ++j) m = fmaxf(m, fabsf(v[k][j]));
    });
    m = group_max<G::LPB>(m);
    if constexpr (G::W > 1) m = block_max<G::W>(m, lds);
    if (bucket_leader<G>()) amax[bk] = m;
}

template <class G, bool EF, class Src>
__global__ void __launch_bounds__(G::THREADS)
k_bucket_absmax(Src src, const float* __restrict__ ef, int64_t n, int64_t nb, float* __restrict__ amax) {
    __shared__ float lds[G::W];
    for (int64_t bk = first_bucket<G>(); bk < nb; bk += bucket_stride<G>()) {
        if ((bk + 1) * (int64_t)G::B <= n)
            absmax_bucket<G, EF, true>(src, ef, n, bk, amax, lds);
        else
            absmax_bucket<G, EF, false>(src, ef, n, bk, amax, lds);
    }
}

template <class G, bool EF, bool FULL, class Src>
__device__ __forceinline__ void int8s_bucket(Src src, float* __restrict__ ef, int64_t n,
                                             int64_t bk, const float* __restrict__ amax,
                                             uint8_t* __restrict__ codes, int64_t pbytes,
                                             float* __restrict__ scale) {
    constexpr int LPB = G::LPB, KH = held_chunks<G>();
    int64_t base = bk * (int64_t)G::B + lane_offset<G>();
    src.prepare(bk * (int64_t)G::B, FULL ? (bk + 1) * (int64_t)G::B : n);
    const float sc = amax[bk] / 127.0f;
    float v[KH][4];
    static_for<0, G::K / KH>([&](auto p) {
        constexpr int P = decltype(p)::value;
        if constexpr (P > 0) part_boundary(base);
        load_chunks<G, P * KH, KH, FULL, EF>(src, ef, base, n, v);
#pragma unroll
        for (int k = 0; k < KH; ++k) {
            const int64_t i = base + (int64_t)(P * KH + k) * LPB * 4;
            uint32_t q[4];
            float e[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int32_t c = 0;
                if (sc != 0.0f) c = (int32_t)fminf(fmaxf(__builtin_rintf(v[k][j] / sc), -127.0f), 127.0f);
                q[j] = (uint32_t)c & 0xFFu;  // masked elements are 0 and give code 0
                e[j] = v[k][j] - (float)c * sc;
            }
            store_codes4<8>(codes, i, pbytes, q);
            if constexpr (EF) store_ef<FULL, 4>(ef, i, n, e);
        }
    });
    if (bucket_leader<G>()) scale[bk] = sc;
}

template <class G, bool EF, class Src>
__global__ void __launch_bounds__(G::THREADS)
k_enc_int8_shared(Src src, float* __restrict__ ef, int64_t n, int64_t nb,
                  const float* __restrict__ amax, uint8_t* __restrict__ codes, int64_t pbytes,
                  float* __restrict__ scale) {
    for (int64_t bk = first_bucket<G>(); bk < nb; bk += bucket_stride<G>()) {
        if ((bk + 1) * (int64_t)G::B <= n)
            int8s_bucket<G, EF, true>(src, ef, n, bk, amax, codes, pbytes, scale);
        else
            int8s_bucket<G, EF, false>(src, ef, n, bk, amax, codes, pbytes, scale);
    }
}

// ============================================================ dispatch
// Geometry per bucket size: LPB lanes per bucket, K chunks per lane, W waves
// per bucket.  A single wave holds up to K = 8 chunks per lane (32 or 64
// values in registers); larger buckets spread over W waves of K = 8, up to
// 16 waves (1,024 threads); 65,536-element buckets take 8 waves of K = 32
// (fp32) or 16 (bf16) chunks, held half at a time (see held_chunks).

template <int E, bool LIST, class F>
hipError_t dispatch_bucket(int32_t bucket, F&& f) {
    const int chunks = bucket / E;
    switch (chunks) {
        case 8: if constexpr (E == 8) return f(Geom<E, 8, 1, 1>{}); break;
        case 16: return f(Geom<E, 16, 1, 1>{});
        case 32: return f(Geom<E, 32, 1, 1>{});
        case 64: return f(Geom<E, 64, 1, 1>{});
        case 128: return f(Geom<E, 64, 2, 1>{});
        case 256: return f(Geom<E, 64, 4, 1>{});
        // E = 8 (bf16 input): one chunk per lane over 8 waves; a whole bucket
        // per wave needed 165 registers (3 waves per SIMD) and measured 5%
        // slower on MI355X
        case 512: if constexpr (E == 8) return f(Geom<E, 64, 1, 8>{}); else return f(Geom<E, 64, 8, 1>{});
        // E = 4, buckets of 4096: two chunks per lane over 8 waves (8 chunks
        // over 2 waves needed 117 registers, 4 waves per SIMD, and measured
        // 5-6% slower on MI355X)
        case 1024: if constexpr (E == 4) return f(Geom<E, 64, 2, 8>{}); else return f(Geom<E, 64, 8, 2>{});
        case 2048: return f(Geom<E, 64, 8, 4>{});
        case 4096: return f(Geom<E, 64, 8, 8>{});
        // 65,536-element buckets (flat arrays only): 8 waves with a
        // 256-register budget per lane, each lane holding half of its chunks
        // at a time.  Holding all of them in 16 waves, these kernels spilled;
        // the tensor-list loads need more registers still (they spilled in
        // every layout tried), so lists stop at 32,768.
        case 8192:
            if constexpr (E == 8 && !LIST) return f(Geom<E, 64, 16, 8>{});
            else if constexpr (E == 4) return f(Geom<E, 64, 8, 16>{});
            break;
        case 16384:
            if constexpr (E == 4 && !LIST) return f(Geom<E, 64, 32, 8>{});
            break;
        default: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace

template <class Src>
struct is_list : std::false_type {};
template <class X>
struct is_list<TensorList<X>> : std::true_type {};

// Calls f(std::true_type) or f(std::false_type): each kernel is compiled
// once with and once without error feedback.
template <class F>
hipError_t with_flag(bool flag, F&& f) {
    return flag ? f(std::true_type{}) : f(std::false_type{});
}

namespace {

template <class Src>
hipError_t launch_uniform_src(Src src, float* ef, int64_t n, int32_t bucket, int32_t bits, bool stochastic,
                              uint64_t seed, uint64_t elem_offset, void* codes, int64_t payload_bytes,
                              float* scale, float* zero, hipStream_t stream) {
    const int64_t nb = (n + bucket - 1) / bucket;
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    return dispatch_bucket<4, is_list<Src>::value>(bucket, [&](auto g) {
        using G = decltype(g);
        const dim3 grid((unsigned)grid_for(nb, G::BPB)), block(G::THREADS);
        return with_flag(ef != nullptr, [&](auto has_ef) {
            constexpr bool EF = decltype(has_ef)::value;
            return with_flag(stochastic, [&](auto is_stoch) {
                constexpr bool ST = decltype(is_stoch)::value;
                if (bits == 8)
                    hipLaunchKernelGGL((k_enc_uniform<G, 8, EF, ST, Src>), grid, block, 0, stream, src, ef, n,
                                       nb, k0, k1, elem_offset, (uint8_t*)codes, payload_bytes, scale, zero);
                else if (bits == 4)
                    hipLaunchKernelGGL((k_enc_uniform<G, 4, EF, ST, Src>), grid, block, 0, stream, src, ef, n,
                                       nb, k0, k1, elem_offset, (uint8_t*)codes, payload_bytes, scale, zero);
                else
                    hipLaunchKernelGGL((k_enc_uniform<G, 2, EF, ST, Src>), grid, block, 0, stream, src, ef, n,
                                       nb, k0, k1, elem_offset, (uint8_t*)codes, payload_bytes, scale, zero);
                return hipGetLastError();
            });
        });
    });
}

template <class Src>
hipError_t launch_ternary_src(Src src, float* ef, int64_t n, int32_t bucket, uint64_t seed, uint64_t elem_offset,
                              uint32_t* words, int64_t payload_bytes, float* scale, hipStream_t stream) {
    const int64_t nb = (n + bucket - 1) / bucket;
    return dispatch_bucket<4, is_list<Src>::value>(bucket, [&](auto g) {
        using G = decltype(g);
        const dim3 grid((unsigned)grid_for(nb, G::BPB)), block(G::THREADS);
        return with_flag(ef != nullptr, [&](auto has_ef) {
            constexpr bool EF = decltype(has_ef)::value;
            hipLaunchKernelGGL((k_enc_ternary<G, EF, Src>), grid, block, 0, stream, src, ef, n, nb, (uint32_t)seed,
                               (uint32_t)(seed >> 32), elem_offset, (uint8_t*)words, payload_bytes, scale);
            return hipGetLastError();
        });
    });
}

template <class Src>
hipError_t launch_qsgd_src(Src src, float* ef, int64_t n, int32_t bucket, uint64_t seed, uint64_t elem_offset,
                           uint32_t* words, int64_t payload_bytes, float* norm, hipStream_t stream) {
    const int64_t nb = (n + bucket - 1) / bucket;
    return dispatch_bucket<4, is_list<Src>::value>(bucket, [&](auto g) {
        using G = decltype(g);
        const dim3 grid((unsigned)grid_for(nb, G::BPB)), block(G::THREADS);
        return with_flag(ef != nullptr, [&](auto has_ef) {
            constexpr bool EF = decltype(has_ef)::value;
            hipLaunchKernelGGL((k_enc_qsgd<G, EF, Src>), grid, block, 0, stream, src, ef, n, nb, (uint32_t)seed,
                               (uint32_t)(seed >> 32), elem_offset, (uint8_t*)words, payload_bytes, norm);
            return hipGetLastError();
        });
    });
}

template <class Src>
hipError_t launch_sign_src(Src src, float* ef, int64_t n, int32_t bucket, uint32_t* words, int64_t payload_bytes,
                           float* scale, hipStream_t stream) {
    const int64_t nb = (n + bucket - 1) / bucket;
    return dispatch_bucket<Src::E, is_list<Src>::value>(bucket, [&](auto g) {
        using G = decltype(g);
        const dim3 grid((unsigned)grid_for(nb, G::BPB)), block(G::THREADS);
        return with_flag(ef != nullptr, [&](auto has_ef) {
            constexpr bool EF = decltype(has_ef)::value;
            hipLaunchKernelGGL((k_enc_sign<G, EF, Src>), grid, block, 0, stream, src, ef, n, nb,
                               (uint8_t*)words, payload_bytes, scale);
            return hipGetLastError();
        });
    });
}

template <class Src>
hipError_t launch_absmax_src(Src src, const float* ef, int64_t n, int32_t bucket, float* amax, hipStream_t stream) {
    const int64_t nb = (n + bucket - 1) / bucket;
    return dispatch_bucket<4, is_list<Src>::value>(bucket, [&](auto g) {
        using G = decltype(g);
        const dim3 grid((unsigned)grid_for(nb, G::BPB)), block(G::THREADS);
        return with_flag(ef != nullptr, [&](auto has_ef) {
            constexpr bool EF = decltype(has_ef)::value;
            hipLaunchKernelGGL((k_bucket_absmax<G, EF, Src>), grid, block, 0, stream, src, ef, n, nb, amax);
            return hipGetLastError();
        });
    });
}

template <class Src>
hipError_t launch_int8_shared_src(Src src, float* ef, int64_t n, int32_t bucket, const float* amax, uint8_t* codes,
                                  int64_t payload_bytes, float* scale, hipStream_t stream) {
    const int64_t nb = (n + bucket - 1) / bucket;
    return dispatch_bucket<4, is_list<Src>::value>(bucket, [&](auto g) {
        using G = decltype(g);
        const dim3 grid((unsigned)grid_for(nb, G::BPB)), block(G::THREADS);
        return with_flag(ef != nullptr, [&](auto has_ef) {
            constexpr bool EF = decltype(has_ef)::value;
            hipLaunchKernelGGL((k_enc_int8_shared<G, EF, Src>), grid, block, 0, stream, src, ef, n, nb, amax, codes,
                               payload_bytes, scale);
            return hipGetLastError();
        });
    });
}

TensorList<float> list_f32(const ListSrc& l) {
    return TensorList<float>{reinterpret_cast<const float* const*>(l.xs), l.offsets, l.seg_first, l.ntensors};
}

}  // namespace

}  // namespace qc
