// k_accumulate.hip -- receive side: acc = (acc or +0) + DQ_0 + ... + DQ_{m-1}
// over m payloads resident in HBM, optionally requantized to uniform codes
// in the same pass.
//
// Each lane owns 16 consecutive elements per chunk (one 16-byte load of
// INT8/FP8 codes per worker, 8 bytes for 4-bit, 4 for 2-bit, 2 for sign) and keeps
// their fp32 sums in registers while it walks the workers in order, so the
// result is bit-identical to adding the decoded terms one worker at a time.
// Two workers' loads are kept in flight while terms are added.  A bucket
// (group) is held by LPB lanes x K chunks x W waves (the layout of
// qc_bucket.hpp with E = 16), which is what the fused requantization needs
// to reduce min/max over the bucket without a second pass over acc.
//
// The per-(worker, bucket) scale and zero are uniform across a wave when a
// bucket spans whole waves; one vector load brings 64 workers' values into
// a register across the wave (see Stats); each worker's pair is then
// copied to vector registers.  2-bit uniform terms read most of their
// decoded values, two at a time, from a per-wave table in LDS; a TernGrad
// term is one fp16-operand fma.  Blocks are mapped to buckets XCD by XCD
// (consecutive buckets on one XCD), so neighbouring buckets' statistics
// share that XCD's L2 lines.
//
// Bounds: a chunk starting below n reads its codes inside the 16-byte
// padded payload (see the payload rules in qc.h).
#include "qc_device.hpp"
#include "qc_bucket.hpp"
#include "qc_launch.hpp"

namespace qc {
namespace {

enum { A_U8 = 0, A_U4 = 1, A_FP8 = 2, A_QSGD = 3, A_SIGN = 4, A_U2 = 5, A_TER = 6 };

// Raw code bits of a 16-element chunk starting at element i of a payload.
template <int F>
struct ChunkBits {
    u32x4 v;
};

template <int F>
__device__ __forceinline__ ChunkBits<F> load_chunk(const uint8_t* __restrict__ p, int64_t i) {
    ChunkBits<F> r;
    if constexpr (F == A_U8 || F == A_FP8) {
        r.v = ld_stream_u4(p + i);
    } else if constexpr (F == A_U4 || F == A_QSGD) {
        const u32x2 h = ld_stream_u2(p + i / 2);
        r.v = u32x4{h.x, h.y, 0u, 0u};
    } else if constexpr (F == A_U2 || F == A_TER) {
        r.v = u32x4{ld_stream_u32(p + i / 4), 0u, 0u, 0u};
    } else {
        const uint32_t h = ld_stream_u16(p + i / 8);
        r.v = u32x4{h, 0u, 0u, 0u};
    }
    return r;
}

// Byte k of a word as fp32 (the compiler turns this into v_cvt_f32_ubyte<k>,
// so the extraction costs nothing).
__device__ __forceinline__ float byte_f(uint32_t w, int k) { return (float)((w >> (8 * k)) & 0xFFu); }

// x & mask through v_bitop3 (truth table 0xC0 = a & b).  The builtin is
// opaque to the optimizer, which would otherwise fold a spread-then-convert
// back into one bitfield extract per code.
__device__ __forceinline__ uint32_t and_mask(uint32_t x, uint32_t mask) {
    return __builtin_amdgcn_bitop3_b32(x, mask, 0u, 0xC0);
}

// m negated (sign bit flipped) when bit `b` of w is set: one shift and one
// v_bitop3 (truth table 0x6C = (a & c) ^ b, c = the sign bit).  Equals
// `bit ? -m : m` for every m.
__device__ __forceinline__ float neg_if_bit(float m, uint32_t w, int b) {
    return __uint_as_float(__builtin_amdgcn_bitop3_b32(w << (31 - b), __float_as_uint(m), 0x80000000u, 0x6C));
}

// a[j] = a[j] + DQ(element j) for the 16 elements of a chunk, each sum
// rounded once in fp32 exactly as decode-then-add would round it.  Sub-byte
// codes are first spread one per byte (a few shifts and masks per word), so
// each code converts with a byte conversion instead of a bitfield extract.
// For QSGD `z` is d = norm/7, for TernGrad s/2.
template <int F>
__device__ __forceinline__ void add_chunk(float (&a)[16], const ChunkBits<F>& c, float s, float z) {
    const uint32_t words[4] = {c.v.x, c.v.y, c.v.z, c.v.w};
    if constexpr (F == A_U8) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float p = byte_f(words[j >> 2], j & 3) * s;
            a[j] = a[j] + (p + z);
        }
    } else if constexpr (F == A_FP8) {
#pragma unroll
        for (int j = 0; j < 16; ++j) a[j] = a[j] + e4m3_decode((words[j >> 2] >> (8 * (j & 3))) & 0xFFu) * s;
    } else if constexpr (F == A_U4) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // nibbles 0,2,4,6 and 1,3,5,7 of the word, one per byte
            const uint32_t sp[2] = {and_mask(words[h], 0x0F0F0F0Fu), and_mask(words[h] >> 4, 0x0F0F0F0Fu)};
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                const float p = byte_f(sp[n & 1], n >> 1) * s;
                a[8 * h + n] = a[8 * h + n] + (p + z);
            }
        }
    } else if constexpr (F == A_U2) {
        uint32_t sp[4];  // sp[r] byte q = code 4q + r
#pragma unroll
        for (int r = 0; r < 4; ++r) sp[r] = and_mask(words[0] >> (2 * r), 0x03030303u);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float p = byte_f(sp[j & 3], j >> 2) * s;
            a[j] = a[j] + (p + z);
        }
    } else if constexpr (F == A_TER) {
        // The term is 0 or +-s, so fma(f, s/2, a) with f in {0, 2, -2} is
        // the exact sum rounded once, as a + DQ is (z = s/2, exact for the
        // scales this path takes).  A 2-bit code is the top two bits of an
        // fp16 number with nothing below them: 0x0000 = +0, 0x4000 = 2,
        // 0xC000 = -2.  One shift and one mask put codes j and j + 8 at the
        // top of the two halves of a word, and each half feeds
        // v_fma_mix_f32 (fp16 operand, fp32 arithmetic) directly: an fma per
        // term and one shift or mask per two terms, against a bitfield
        // extract, a conversion and an fma.
        //
        // The never-emitted code 2 decodes to +0 but reads here as 0x8000 =
        // -0, and acc + -0 differs from acc + +0 only when acc is -0 (-0
        // against +0).  From there on the two sums either agree bit for bit
        // or are -0 here and +0 by the rule (a sum is -0 only as -0 + -0;
        // every other term makes both sums equal), so a sum that ends at
        // anything but -0 is the rule's sum, and the few that end at -0 are
        // summed again term by term after the last worker.
        const uint32_t w = words[0];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const h16x2 f = __builtin_bit_cast(h16x2, (w << (14 - 2 * j)) & 0xC000C000u);
            a[j] = __builtin_fmaf((float)f.x, z, a[j]);
            a[j + 8] = __builtin_fmaf((float)f.y, z, a[j + 8]);
        }
    } else if constexpr (F == A_QSGD) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t sp[2] = {and_mask(words[h], 0x0F0F0F0Fu), and_mask(words[h] >> 4, 0x0F0F0F0Fu)};
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint32_t lv = and_mask(sp[e], 0x07070707u);
                // sign bits (bit 3 of each byte) kept only where the level is
                // nonzero: level 0 decodes to +0 whatever its sign bit
                const uint32_t nz = ((lv + 0x7F7F7F7Fu) & 0x80808080u) >> 4;
                const uint32_t sg = sp[e] & nz;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float mag = byte_f(lv, q) * z;
                    const int j = 8 * h + 2 * q + e;
                    a[j] = a[j] + neg_if_bit(mag, sg, 8 * q + 3);
                }
            }
        }
    } else {
        // sign: DQ = bit ? -s : s
#pragma unroll
        for (int j = 0; j < 16; ++j) a[j] = a[j] + neg_if_bit(s, words[0], j);
    }
}

// The fast forms above rely on 0 * s being +0: for TernGrad's s and QSGD's
// d that holds when the value is +0 or positive and finite (TernGrad's also
// on s/2 being exact, which rules out subnormal and tiny normal scales).
// Otherwise (an overflowed sum of squares gives d = inf; a caller may pass
// anything) the worker's terms are decoded one by one exactly as the decoder
// does.
template <int F>
__device__ __forceinline__ bool needs_exact_path(float s, float z) {
    if constexpr (F == A_QSGD) return __float_as_uint(z) >= 0x7F800000u;
    else if constexpr (F == A_TER) {
        // the fast form also needs s/2 exact: s = +0 or s >= 2^-125
        const uint32_t b = __float_as_uint(s);
        return b >= 0x7F800000u || b - 1u < 0x00FFFFFFu;
    }
    else return false;
}

template <int F>
__device__ __forceinline__ void add_chunk_exact(float (&a)[16], const ChunkBits<F>& c, float s, float z) {
    const uint32_t w[2] = {c.v.x, c.v.y};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        float t;
        if constexpr (F == A_QSGD) {
            const uint32_t code = (w[j >> 3] >> (4 * (j & 7))) & 0xFu;
            const uint32_t level = code & 7u;
            const float mag = (float)level * z;
            t = level == 0u ? 0.0f : ((code & 8u) ? -mag : mag);
        } else {
            const uint32_t code = (w[0] >> (2 * j)) & 0x3u;
            t = (code & 1u) ? ((code & 2u) ? -s : s) : 0.0f;
        }
        a[j] = a[j] + t;
    }
}

// One TernGrad sum (element idx of statistics group gb), one term at a
// time exactly as the decoder's rule gives them.
__device__ __noinline__ float ter_sum_one(const uint8_t* __restrict__ codes, int64_t pbytes,
                                          const float* __restrict__ scale, int64_t ng, int64_t gb, int32_t m,
                                          int64_t idx, const float* __restrict__ acc, int32_t accumulate) {
    float r = accumulate ? acc[idx] : 0.0f;
    for (int32_t w = 0; w < m; ++w) {
        const uint32_t code = (codes[(int64_t)w * pbytes + idx / 4] >> (2 * (idx % 4))) & 3u;
        const float s = scale[(int64_t)w * ng + gb];
        r = r + ((code & 1u) ? ((code & 2u) ? -s : s) : 0.0f);
    }
    return r;
}

// 2-bit uniform codes through a per-wave table in LDS.  A 2-bit code has
// four decoded values per (worker, bucket), so two adjacent codes have 16;
// per worker, lanes 0-31 write the 16 pairs (d(c0), d(c1)) of decoded
// values, each computed exactly as the decoder computes it, to the wave's
// 256-byte-aligned table, entry c0 + 4 c1 at byte 8 (c0 + 4 c1).  A pair of
// terms is then one v_perm (the pair's 4 code bits, times 8, as the low
// address byte over the table's base), one ds_read_b64 and two adds, where
// the arithmetic path takes a conversion, a multiply and two adds per term.
// The LDS pipe delivers 32 such terms per CU clock and works beside the
// VALU, which bounds 2-bit sums, so 12 of a chunk's 16 terms (the pairs
// 4q+2, 4q+3 and, for q < 2, 4q, 4q+1) go through the table and 4 (codes 8,
// 9, 12 and 13) through the arithmetic.  Measured on the 64-worker sum of
// 2^26 elements in buckets of 2,048 with requantization: 417 us
// all-arithmetic (statistics in scalar registers), 383 us with them in
// vector registers, 355 us with 12 terms through a one-code table (a v_perm
// and a ds_read_b32 per term; 397 us with all 16).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) f32x2 lds_f32x2;
__device__ __forceinline__ uint32_t lds_addr(float* p) { return (uint32_t)(uintptr_t)(lds_f32*)p; }
__device__ __forceinline__ f32x2 lds_load2(uint32_t a) { return *(const lds_f32x2*)(uintptr_t)a; }
__device__ __forceinline__ void lds_store(uint32_t a, float v) { *(lds_f32*)(uintptr_t)a = v; }

// lanes 0-31: float l of the pair table, d(c) for c = code (l & 1 ? 1 : 0) of entry l >> 1
__device__ __forceinline__ void u2_pair_table_store(uint32_t tbase, float s, float z) {
    const uint32_t l = (uint32_t)lane_id();
    if (l < 32u) {
        const uint32_t c = (l & 1u) ? (l >> 3) : ((l >> 1) & 3u);
        const float p = (float)c * s;
        lds_store(tbase + 4u * l, p + z);
    }
}

__device__ __forceinline__ void add_chunk_u2_pairs(float (&a)[16], uint32_t w, float s, float z, uint32_t tbase) {
    const uint32_t p01 = and_mask(w << 3, 0x78787878u);  // byte q = 8 (c(4q) + 4 c(4q+1))
    const uint32_t p23 = and_mask(w >> 1, 0x78787878u);  // byte q = 8 (c(4q+2) + 4 c(4q+3))
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const f32x2 v = lds_load2(__builtin_amdgcn_perm(tbase, p23, 0x07060500u | (uint32_t)q));
        a[4 * q + 2] = a[4 * q + 2] + v.x;
        a[4 * q + 3] = a[4 * q + 3] + v.y;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const f32x2 v = lds_load2(__builtin_amdgcn_perm(tbase, p01, 0x07060500u | (uint32_t)q));
        a[4 * q] = a[4 * q] + v.x;
        a[4 * q + 1] = a[4 * q + 1] + v.y;
    }
    const uint32_t s0 = and_mask(w, 0x03030303u);       // byte q = c(4q)
    const uint32_t s1 = and_mask(w >> 2, 0x03030303u);  // byte q = c(4q+1)
#pragma unroll
    for (int q = 2; q < 4; ++q) {
        const float p0 = byte_f(s0, q) * s;
        a[4 * q] = a[4 * q] + (p0 + z);
        const float p1 = byte_f(s1, q) * s;
        a[4 * q + 1] = a[4 * q + 1] + (p1 + z);
    }
}

constexpr bool has_zero(int F) { return F == A_U8 || F == A_U4 || F == A_U2; }

// Per-(worker, bucket) statistics.  When a bucket spans whole waves they are
// wave-uniform: lane l loads worker c0+l's scale and zero (one vector load
// per 64 workers) and worker w's pair is taken with v_readlane.  (Reading
// them through the scalar cache instead stalls every pipeline step: scalar
// loads complete out of order, so the compiler can only wait for all of
// them, including the next group's.)  Buckets narrower than a wave load each
// worker's pair per lane, as ordinary in-order vector loads.
template <class G, int F>
struct Stats {
    static constexpr bool WAVE_UNIFORM = G::LPB == WAVE;
    float ls = 0.0f, lz = 0.0f;  // this lane's worker (c0 + lane), wave-uniform case
    int32_t c0 = 0;

    __device__ __forceinline__ void load_chunk_of_workers(const float* __restrict__ scale,
                                                          const float* __restrict__ zero, int64_t nb,
                                                          int64_t bk, int32_t first, int32_t end) {
        if constexpr (WAVE_UNIFORM) {
            c0 = first;
            const int32_t w = first + lane_id();
            ls = 0.0f;
            lz = 0.0f;
            if (w < end) {
                ls = scale[(int64_t)w * nb + bk];
                if constexpr (has_zero(F)) lz = zero[(int64_t)w * nb + bk];
            }
        }
    }

    __device__ __forceinline__ void get(const float* __restrict__ scale, const float* __restrict__ zero,
                                        int64_t nb, int64_t bk, int32_t w, float& s, float& z) const {
        if constexpr (WAVE_UNIFORM) {
            s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls), w - c0));
            z = has_zero(F) ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lz), w - c0)) : 0.0f;
        } else {
            s = scale[(int64_t)w * nb + bk];
            z = has_zero(F) ? zero[(int64_t)w * nb + bk] : 0.0f;
        }
    }
};

// Loads of worker w's code chunks for one bucket.
template <class G, int F, bool FULL>
__device__ __forceinline__ void load_codes(const uint8_t* __restrict__ codes, int64_t pbytes, int64_t base,
                                           int64_t n, int32_t w, ChunkBits<F> (&c)[G::K]) {
    const uint8_t* pw = codes + (int64_t)w * pbytes;
#pragma unroll
    for (int k = 0; k < G::K; ++k) {
        const int64_t i = base + (int64_t)k * G::LPB * 16;
        if (FULL || i < n) c[k] = load_chunk<F>(pw, i);
        else c[k].v = u32x4{0u, 0u, 0u, 0u};
    }
}

// Tile bk of G::B elements, inside statistics group gb of ng groups (a tile
// is the whole group, or a part of it for the largest groups).
template <class G, int F, int RQBITS, bool RQ, bool FULL>
__device__ __forceinline__ void acc_bucket(const uint8_t* __restrict__ codes, const float* __restrict__ scale,
                                           const float* __restrict__ zero, int32_t m, int64_t n, int64_t ng,
                                           int64_t pbytes, float* __restrict__ acc, int32_t accumulate,
                                           uint8_t* __restrict__ rq_codes, int64_t rq_pbytes,
                                           float* __restrict__ rq_scale, float* __restrict__ rq_zero,
                                           int64_t bk, int64_t gb, float* lds, uint32_t tbase, float* xw) {
    constexpr int K = G::K, LPB = G::LPB, UW = 2;
    constexpr bool TAB = F == A_U2 && Stats<G, F>::WAVE_UNIFORM;
    const int64_t base = bk * (int64_t)G::B + lane_offset<G>();

    float a[K][16];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int64_t i = base + (int64_t)k * LPB * 16;
#pragma unroll
        for (int j = 0; j < 16; ++j) a[k][j] = 0.0f;
        if (accumulate) {
            if (FULL || i + 16 <= n) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 t = ld_stream_f4(acc + i + 4 * q);
                    a[k][4 * q] = t.x; a[k][4 * q + 1] = t.y;
                    a[k][4 * q + 2] = t.z; a[k][4 * q + 3] = t.w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (i + j < n) a[k][j] = acc[i + j];
            }
        }
    }

    // Workers are taken 64 at a time (the statistics of one chunk of workers
    // fit one register across the wave).  Within a chunk UW register slots
    // form a rolling prefetch: as soon as worker w's terms have been added
    // (in worker order), its slot is refilled with worker w+UW, so every wave
    // always has UW workers' code loads in flight while it computes.  The
    // steady-state loop takes UW workers at a time and holds no branch (with the
    // adds under a condition, the compiler moved each refill into the
    // conditional block that used it, right before its wait), and a
    // scheduling barrier after each refill keeps the instruction scheduler
    // from moving it down next to its use to shorten register live ranges:
    // either way the prefetch was lost.  The last (chunk size % UW) workers
    // are added after the loop, from the slots that already hold them.
    // Refills clamp the worker index to the chunk's last worker; the
    // repeated loads past the end are never added.
    constexpr int32_t CHUNK = Stats<G, F>::WAVE_UNIFORM ? WAVE : 0x7FFFFFFF;
    Stats<G, F> st;
    auto add_worker = [&](int32_t w, const ChunkBits<F> (&c)[K]) {
        float s, z;
        st.get(scale, zero, ng, gb, w, s, z);
        if constexpr (F == A_QSGD) z = s / 7.0f;
        if constexpr (F == A_TER) z = s * 0.5f;
        const bool exact = needs_exact_path<F>(s, z);
        // Wave-uniform statistics arrive in scalar registers (v_readlane).
        // On gfx950 a VALU op that reads a scalar register issues at about
        // half the rate of one whose operands are all vector registers
        // (measured: v_add_f32 38 vs 67 T lane-ops/s), and the term loop is
        // VALU-bound for sub-byte codes, so s and z are copied to vector
        // registers once per worker.
        if constexpr (Stats<G, F>::WAVE_UNIFORM) asm volatile("" : "+v"(s), "+v"(z));
        if (exact) {
            if constexpr (F == A_QSGD || F == A_TER) {
#pragma unroll
                for (int k = 0; k < K; ++k) add_chunk_exact<F>(a[k], c[k], s, z);
            }
        } else if constexpr (TAB) {
            u2_pair_table_store(tbase, s, z);
#pragma unroll
            for (int k = 0; k < K; ++k) add_chunk_u2_pairs(a[k], c[k].v.x, s, z, tbase);
        } else {
#pragma unroll
            for (int k = 0; k < K; ++k) add_chunk<F>(a[k], c[k], s, z);
        }
    };
    for (int32_t c0 = 0; c0 < m; c0 += CHUNK) {
        const int32_t cend = m - c0 > CHUNK ? c0 + CHUNK : m;
        const int32_t last = cend - 1;
        st.load_chunk_of_workers(scale, zero, ng, gb, c0, cend);
        ChunkBits<F> slot[UW][K];
#pragma unroll
        for (int u = 0; u < UW; ++u)
            load_codes<G, F, FULL>(codes, pbytes, base, n, c0 + u < last ? c0 + u : last, slot[u]);
        int32_t w0 = c0;
        for (; w0 + UW <= cend; w0 += UW) {
#pragma unroll
            for (int u = 0; u < UW; ++u) {
                add_worker(w0 + u, slot[u]);
                const int32_t w = w0 + u + UW;
                load_codes<G, F, FULL>(codes, pbytes, base, n, w < last ? w : last, slot[u]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int u = 0; u < UW - 1; ++u)
            if (w0 + u < cend) add_worker(w0 + u, slot[u]);
    }

    // TernGrad sums ending at -0 (see add_chunk): summed again term by term
    if constexpr (F == A_TER) {
        bool negz = false;
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int j = 0; j < 16; ++j) negz |= __float_as_uint(a[k][j]) == 0x80000000u;
        if (__any(negz)) {
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (__float_as_uint(a[k][j]) == 0x80000000u)
                        a[k][j] = ter_sum_one(codes, pbytes, scale, ng, gb, m,
                                              base + (int64_t)k * LPB * 16 + j, acc, accumulate);
        }
    }

    // A lane's 16 sums are 64 contiguous bytes: full tiles of whole-wave
    // buckets store each chunk's 4 KiB span through the wave's LDS buffer
    // (store_wave_span16: 1 KiB-contiguous streaming stores).  Not for the
    // 2-bit sum with requantization: the buffer's addresses took it from
    // 127 to 131 registers and 4 to 3 waves per SIMD, 11% slower; the
    // others gained 4-6%.
    if constexpr (FULL && LPB == WAVE && !(F == A_U2 && RQ)) {
        const int64_t c0 = bk * (int64_t)G::B + (G::W > 1 ? (int64_t)wave_id() * G::SUB : 0);
#pragma unroll
        for (int k = 0; k < K; ++k) store_wave_span16(acc + c0 + (int64_t)k * LPB * 16, a[k], xw);
    } else {
    // Otherwise acc is written with plain stores, which L2 merges into whole
    // lines (streaming stores would not be merged).
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int64_t i = base + (int64_t)k * LPB * 16;
        if (FULL || i + 16 <= n) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<f32x4*>(acc + i + 4 * q) =
                    f32x4{a[k][4 * q], a[k][4 * q + 1], a[k][4 * q + 2], a[k][4 * q + 3]};
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (i + j < n) acc[i + j] = a[k][j];
        }
    }
    }

    if constexpr (RQ) {
        // requantize the bucket's sums: the uniform rule with no feedback
        constexpr uint32_t L = (1u << RQBITS) - 1u;
        float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (FULL || base + (int64_t)k * LPB * 16 + j < n) {
                    mn = fminf(mn, a[k][j]);
                    mx = fmaxf(mx, a[k][j]);
                }
        mn = group_min<LPB>(mn);
        mx = group_max<LPB>(mx);
        if constexpr (G::W > 1) {
            mn = block_min<G::W>(mn, lds);
            mx = block_max<G::W>(mx, lds);
        }
        mn = mn + 0.0f;
        mx = mx + 0.0f;
        const float sc = (mx - mn) / (float)L;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t i = base + (int64_t)k * LPB * 16;
            uint32_t q[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                uint32_t cq = 0;
                if (sc != 0.0f) {
                    const float t = (a[k][j] - mn) / sc;
                    cq = (uint32_t)fminf(fmaxf(__builtin_rintf(t), 0.0f), (float)L);
                }
                q[j] = (FULL || i + j < n) ? cq : 0u;
            }
            if constexpr (RQBITS == 8) {
                u32x4 o;
                o.x = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
                o.y = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
                o.z = q[8] | (q[9] << 8) | (q[10] << 16) | (q[11] << 24);
                o.w = q[12] | (q[13] << 8) | (q[14] << 16) | (q[15] << 24);
                if (FULL || i < rq_pbytes) st_u4(rq_codes + i, o);
            } else if constexpr (RQBITS == 4) {
                uint32_t lo = 0, hi = 0;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    lo |= q[j] << (4 * j);
                    hi |= q[8 + j] << (4 * j);
                }
                if (FULL || i / 2 < rq_pbytes) {
                    st_u32(rq_codes + i / 2, lo);
                    st_u32(rq_codes + i / 2 + 4, hi);
                }
            } else {
                uint32_t word = 0;
#pragma unroll
                for (int j = 0; j < 16; ++j) word |= q[j] << (2 * j);
                if (FULL || i / 4 < rq_pbytes) st_u32(rq_codes + i / 4, word);
            }
        }
        if (bucket_leader<G>()) {
            rq_scale[bk] = sc;
            rq_zero[bk] = mn;
        }
    }
}

// nb tiles of G::B elements; tile bk belongs to statistics group
// bk >> tshift of ng (tshift = 0 when a tile is a whole group, which
// requantization requires).
// TernGrad sums of whole-wave buckets with up to 2 chunks per lane fit 5
// waves per SIMD (94 registers) when asked to; left alone the compiler
// takes 98 and 4 waves, 3-4% slower on 64 x 2^26 in buckets of 2,048.  (Six
// waves spill; so do 4-chunk buckets at five.)
template <int F, class G>
constexpr int min_waves() { return F == A_TER && G::LPB == WAVE && G::K <= 2 ? 5 : 1; }

template <class G, int F, int RQBITS, bool RQ>
__global__ void __launch_bounds__(G::THREADS, (min_waves<F, G>()))
k_dequant_acc(const uint8_t* __restrict__ codes, const float* __restrict__ scale,
              const float* __restrict__ zero, int32_t m, int64_t n, int64_t nb, int64_t ng, int32_t tshift,
              int64_t pbytes, float* __restrict__ acc, int32_t accumulate, uint8_t* __restrict__ rq_codes,
              int64_t rq_pbytes, float* __restrict__ rq_scale, float* __restrict__ rq_zero) {
    __shared__ float lds[G::W];
    // one 256-byte-aligned decode table per wave (2-bit uniform codes; the
    // array is dropped from kernels that do not read it)
    __shared__ __align__(256) float tab[G::THREADS / WAVE][64];
    const uint32_t tbase = lds_addr(&tab[wave_id()][0]);
    // one 4 KiB buffer per wave for the sums' contiguous stores
    __shared__ __align__(16) float xbuf[G::THREADS / WAVE][G::LPB == WAVE ? 1024 : 4];
    float* xw = &xbuf[wave_id()][0];

    // XCD-aware order: blocks are dispatched round-robin over the 8 XCDs,
    // so block b runs on XCD b%8; give each XCD a contiguous bucket range.
    const int64_t nblk = gridDim.x;
    const int64_t per_xcd = (nblk + 7) / 8;
    const int64_t vblock = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (vblock * G::BPB >= nb) return;  // spare blocks when gridDim.x % 8 != 0

    const int64_t first = G::W > 1 ? vblock
                                   : vblock * G::BPB + wave_id() * G::GROUPS + lane_id() / G::LPB;
    for (int64_t bk = first; bk < nb; bk += per_xcd * 8 * G::BPB) {
        int64_t bks = bk;
        // a bucket spanning whole waves has a wave-uniform index: keep it in
        // scalar registers so per-worker statistics come through the scalar cache
        if constexpr (G::LPB == WAVE) bks = __builtin_amdgcn_readfirstlane((int)bk);
        const int64_t gb = bks >> tshift;
        if ((bks + 1) * (int64_t)G::B <= n)
            acc_bucket<G, F, RQBITS, RQ, true>(codes, scale, zero, m, n, ng, pbytes, acc, accumulate,
                                               rq_codes, rq_pbytes, rq_scale, rq_zero, bks, gb, lds, tbase, xw);
        else
            acc_bucket<G, F, RQBITS, RQ, false>(codes, scale, zero, m, n, ng, pbytes, acc, accumulate,
                                                rq_codes, rq_pbytes, rq_scale, rq_zero, bks, gb, lds, tbase, xw);
    }
}

// Bucket of `group` elements as LPB lanes x K chunks of 16 x W waves: whole
// waves with up to 4 chunks per lane before spreading over more waves.
// 65,536-element groups (and FP8 rows of 32,768) are summed in tiles of
// 16,384 elements, each reading its group's statistics: holding a whole
// group, those kernels spilled to scratch memory (64 sums per lane in a
// 1,024-thread block; FP8's decode on top of 64 sums in a 512-thread one).
template <int F, class Fn>
hipError_t dispatch_group(int32_t group, Fn&& fn) {
    switch (group / 16) {
        case 4: return fn(Geom<16, 4, 1, 1>{});
        case 8: return fn(Geom<16, 8, 1, 1>{});
        case 16: return fn(Geom<16, 16, 1, 1>{});
        case 32: return fn(Geom<16, 32, 1, 1>{});
        case 64: return fn(Geom<16, 64, 1, 1>{});
        case 128: return fn(Geom<16, 64, 2, 1>{});
        case 256: return fn(Geom<16, 64, 4, 1>{});
        case 512: return fn(Geom<16, 64, 4, 2>{});
        case 1024: return fn(Geom<16, 64, 4, 4>{});
        case 2048:
            if constexpr (F == A_FP8) return fn(Geom<16, 64, 4, 4>{});
            else return fn(Geom<16, 64, 4, 8>{});
        case 4096: return fn(Geom<16, 64, 4, 4>{});
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_encode_requant(const float* acc, int64_t n, int32_t group, int32_t bits, void* rq_codes,
                                 float* rq_scale, float* rq_zero, hipStream_t stream) {
    const int64_t code_bytes = bits == 8 ? n : (bits == 4 ? (n + 7) / 8 * 4 : (n + 15) / 16 * 4);
    return launch_encode_uniform(acc, nullptr, n, group, bits, false, 0, 0, rq_codes, (code_bytes + 15) / 16 * 16,
                                 rq_scale, rq_zero, stream);
}

template <int F>
hipError_t launch_fmt(const void* codes, const float* scale, const float* zero, int32_t m, int64_t n,
                      int32_t group, int32_t bits, int64_t pbytes, float* acc, bool accumulate,
                      void* rq_codes, float* rq_scale, float* rq_zero, hipStream_t stream) {
    const int64_t ng = (n + group - 1) / group;
    return dispatch_group<F>(group, [&](auto g) {
        using G = decltype(g);
        const int32_t tshift = log2_exact(group / G::B);
        const int64_t nt = (n + G::B - 1) / G::B;
        int64_t blocks = grid_for(nt, G::BPB);
        blocks = (blocks + 7) / 8 * 8;  // whole rounds over the 8 XCDs
        const dim3 grid((unsigned)blocks), block(G::THREADS);
        const int64_t rq_code_bytes = bits == 8 ? n : (bits == 4 ? (n + 7) / 8 * 4 : (n + 15) / 16 * 4);
        const int64_t rq_pbytes = (rq_code_bytes + 15) / 16 * 16;
        if (rq_codes == nullptr || tshift > 0) {
            hipLaunchKernelGGL((k_dequant_acc<G, F, 8, false>), grid, block, 0, stream,
                               (const uint8_t*)codes, scale, zero, m, n, nt, ng, tshift, pbytes, acc,
                               (int32_t)accumulate, (uint8_t*)nullptr, (int64_t)0, (float*)nullptr,
                               (float*)nullptr);
            if (rq_codes == nullptr) return hipGetLastError();
            if constexpr (F == A_U8 || F == A_U4 || F == A_U2) {
                // tiles smaller than the group: the sums are requantized by
                // the uniform encoder in a second launch (the same rule,
                // without error feedback), reading them back once
                const hipError_t e = hipGetLastError();
                if (e != hipSuccess) return e;
                return launch_encode_requant(acc, n, group, bits, rq_codes, rq_scale, rq_zero, stream);
            } else {
                return hipErrorInvalidValue;
            }
        } else if constexpr (F == A_U8 || F == A_U4 || F == A_U2) {
            // requantization to the input's own bit width
            constexpr int RQB = F == A_U8 ? 8 : (F == A_U4 ? 4 : 2);
            hipLaunchKernelGGL((k_dequant_acc<G, F, RQB, true>), grid, block, 0, stream,
                               (const uint8_t*)codes, scale, zero, m, n, nt, ng, tshift, pbytes, acc,
                               (int32_t)accumulate, (uint8_t*)rq_codes, rq_pbytes, rq_scale, rq_zero);
        } else {
            return hipErrorInvalidValue;
        }
        return hipGetLastError();
    });
}

}  // namespace

hipError_t launch_dequant_accumulate(int32_t fmt, const void* codes, const float* scale,
                                     const float* zero, int32_t m, int64_t n, int32_t group,
                                     int32_t bits, int64_t payload_bytes, float* acc,
                                     bool accumulate, void* rq_codes, float* rq_scale,
                                     float* rq_zero, hipStream_t stream) {
    switch (fmt) {
        case 0:
            if (bits == 8)
                return launch_fmt<A_U8>(codes, scale, zero, m, n, group, bits, payload_bytes, acc,
                                        accumulate, rq_codes, rq_scale, rq_zero, stream);
            if (bits == 4)
                return launch_fmt<A_U4>(codes, scale, zero, m, n, group, bits, payload_bytes, acc,
                                        accumulate, rq_codes, rq_scale, rq_zero, stream);
            return launch_fmt<A_U2>(codes, scale, zero, m, n, group, bits, payload_bytes, acc,
                                    accumulate, rq_codes, rq_scale, rq_zero, stream);
        case 1:
            return launch_fmt<A_FP8>(codes, scale, zero, m, n, group, bits, payload_bytes, acc,
                                     accumulate, rq_codes, rq_scale, rq_zero, stream);
        case 2:
            return launch_fmt<A_QSGD>(codes, scale, zero, m, n, group, bits, payload_bytes, acc,
                                      accumulate, rq_codes, rq_scale, rq_zero, stream);
        case 4:
            return launch_fmt<A_TER>(codes, scale, zero, m, n, group, bits, payload_bytes, acc,
                                     accumulate, rq_codes, rq_scale, rq_zero, stream);
        default:
            return launch_fmt<A_SIGN>(codes, scale, zero, m, n, group, bits, payload_bytes, acc,
                                      accumulate, rq_codes, rq_scale, rq_zero, stream);
    }
}

}  // namespace qc
