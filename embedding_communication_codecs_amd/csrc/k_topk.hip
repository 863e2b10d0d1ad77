// k_topk.hip -- top-k sparsification with error feedback, its decoder and
// the receive-side sum of several workers' sparse payloads.
//
// Encoder: one block per bucket.  Thread t holds EPT consecutive elements
// of the bucket in registers (v = ef + x, read from one array or in place
// from a list of tensors).  The k-th largest magnitude key
// (the fp32 bits with the sign cleared, which order like |v|) is found
// exactly.  For k up to KSMALL: tau, the k-th largest of the threads'
// maxima, bounds it from below (k threads hold an element at or above tau),
// the few elements at or above tau are gathered in LDS and one wave picks
// the k-th largest among them.  Otherwise, or when too many elements pass
// tau: a most-significant-digit radix select, four passes over the 31 key
// bits (8, 8, 8 and 7 bits), each building an LDS histogram of the next
// digit among the elements that match the digits fixed so far.  Then every
// element with a larger key is sent, and of those equal to the threshold
// the ones with the smallest indices, as many as are still needed.  One
// block-wide exclusive scan of (larger, equal) counts gives every sent
// element its slot, so the pairs come out in index order.  Buckets of
// 16,384 to 65,536 take 1,024-thread blocks whose lanes cannot hold 16 to 64
// values each in registers: they take the radix select only, reading the
// bucket again (from L2 or the last-level cache) for every pass.
//
// Decoder and sum: the bucket's span of the dense output is held in LDS
// (zeros, or the caller's values for a continued sum) while the pairs are
// placed or added, then written out in one pass; buckets above 8,192 are
// handled in tiles of 8,192 elements, each scanning all of the bucket's
// pairs and applying those that fall in it.  The decoder and the sum
// for k >= 64 give each bucket a block; the sum for smaller k gives it one
// wave, which orders the workers' additions to one index without barriers
// (owner tags in LDS, then worker by worker for whatever is left).
#include "qc_device.hpp"
#include "qc_bucket.hpp"
#include "qc_launch.hpp"
#include "k_encode.hpp"  // the input sources (one array, or a tensor list)

#include <atomic>

namespace qc {
namespace {

constexpr uint32_t kNoIndex = 0xFFFFFFFFu;
constexpr int KSMALL = 16;  // k up to this takes the candidate path

__device__ __forceinline__ uint32_t mag_key(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// Block-wide exclusive scan of two counters (thread order), with the block
// totals; `lds` holds 2 * (T/64) values.  Ends with a barrier, so lds can
// be reused.
template <int T>
__device__ __forceinline__ void block_exclusive_scan2(uint32_t a, uint32_t b, uint32_t& ea, uint32_t& eb,
                                                      uint32_t& ta, uint32_t& tb, uint32_t* lds) {
    constexpr int NW = T / WAVE;
    uint32_t ia = a, ib = b;  // inclusive scans inside the wave
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
        const uint32_t ua = (uint32_t)__shfl_up((int)ia, off, WAVE);
        const uint32_t ub = (uint32_t)__shfl_up((int)ib, off, WAVE);
        if (lane_id() >= off) {
            ia += ua;
            ib += ub;
        }
    }
    if constexpr (NW > 1) {
        if (lane_id() == WAVE - 1) {
            lds[wave_id()] = ia;
            lds[NW + wave_id()] = ib;
        }
        __syncthreads();
        uint32_t pa = 0, pb = 0, sa = 0, sb = 0;
        for (int w = 0; w < NW; ++w) {
            if (w < wave_id()) {
                pa += lds[w];
                pb += lds[NW + w];
            }
            sa += lds[w];
            sb += lds[NW + w];
        }
        __syncthreads();
        ea = pa + ia - a;
        eb = pb + ib - b;
        ta = sa;
        tb = sb;
    } else {
        ea = ia - a;
        eb = ib - b;
        ta = (uint32_t)__shfl((int)ia, WAVE - 1, WAVE);
        tb = (uint32_t)__shfl((int)ib, WAVE - 1, WAVE);
    }
}

// Maximum over the wave, returned wave-uniform; all 64 lanes must be
// active.  DPP moves combine lanes inside each row of 16 (swap neighbours,
// swap pairs, mirror each half row, mirror the row), then the four row
// maxima are read out with v_readlane.
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));  // row_mirror
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return umax(umax(r0, r1), umax(r2, r3));
}

// The r-th largest (r = 1..K) of the values held by a wave, Q per lane,
// counted with multiplicity; values are encoded key+1, 0 meaning "none".
// Returns 0 if the wave holds fewer than r values.  Destroys c.
template <int Q>
__device__ __forceinline__ uint32_t wave_rth_largest(uint32_t (&c)[Q], uint32_t r) {
    uint32_t m = 0;
    for (uint32_t it = 0; it < r; ++it) {
        uint32_t best = 0;
#pragma unroll
        for (int q = 0; q < Q; ++q) best = c[q] > best ? c[q] : best;
        m = wave_max_u32(best);
        if (m == 0) break;  // fewer than r values (wave-uniform)
        // one occurrence is removed: the first lane holding it, its first slot
        const uint64_t holders = __ballot(best == m);
        if (lane_id() == __builtin_ctzll(holders)) {
            bool done = false;
#pragma unroll
            for (int q = 0; q < Q; ++q)
                if (!done && c[q] == m) {
                    c[q] = 0;
                    done = true;
                }
        }
    }
    return m;
}

// Exclusive scan over the wave (lane order) and the wave total.
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t a, uint32_t& total) {
    uint32_t i = a;
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
        const uint32_t t = (uint32_t)__shfl_up((int)i, off, WAVE);
        if (lane_id() >= off) i += t;
    }
    total = (uint32_t)__shfl((int)i, WAVE - 1, WAVE);
    return i - a;
}

// v[e] = ef + x for the EPT elements from global index i0 (0 at or past n).
template <bool EF>
__device__ __forceinline__ float load_one(const FlatX& s, const float* __restrict__ ef, int64_t i, int64_t n) {
    if (i >= n) return 0.0f;
    const float g = s.x[i];
    return EF ? ef[i] + g : g;
}
template <bool EF>
__device__ __forceinline__ float load_one(const TensorList<float>& s, const float* __restrict__ ef, int64_t i,
                                          int64_t n) {
    if (i >= n) return 0.0f;
    int32_t t = s.lo;
    const float g = s.elem(t, i);
    return EF ? ef[i] + g : g;
}
template <int EPT, bool EF, class Src>
__device__ __forceinline__ void load_elems(const Src& src, const float* __restrict__ ef, int64_t i0, int64_t n,
                                           bool full, float (&v)[EPT]) {
    if constexpr (EPT % 4 == 0 && std::is_same<Src, FlatX>::value) {
        // plain (not streaming) loads: the residual is written back to the
        // same lines right after the selection
        if (full) {
#pragma unroll
            for (int q = 0; q < EPT / 4; ++q) {
                f32x4 g = ld_f4(src.x + i0 + 4 * q);
                if constexpr (EF) g = ld_f4(ef + i0 + 4 * q) + g;
                v[4 * q] = g.x; v[4 * q + 1] = g.y; v[4 * q + 2] = g.z; v[4 * q + 3] = g.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < EPT; ++e) v[e] = load_one<EF>(src, ef, i0 + e, n);
        }
    } else if constexpr (EPT % 4 == 0) {
#pragma unroll
        for (int q = 0; q < EPT / 4; ++q) {
            float t[4];
            if (full) src.template load<true, EF>(ef, i0 + 4 * q, n, t);
            else src.template load<false, EF>(ef, i0 + 4 * q, n, t);
            v[4 * q] = t[0]; v[4 * q + 1] = t[1]; v[4 * q + 2] = t[2]; v[4 * q + 3] = t[3];
        }
    } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e) v[e] = load_one<EF>(src, ef, i0 + e, n);
    }
}

// One digit of the most-significant-digit radix select.  hist holds the
// counts of the next digit (bits shift.. under dmask) among the elements
// whose key matches prefix under pmask; krem of them are still to be
// selected.  Wave 0 finds the digit d whose suffix count (bins >= d) first
// reaches krem, and every thread fixes d in prefix and takes the count of
// the larger bins off krem.  Ends with a barrier (bcast and hist are free).
template <int T>
__device__ __forceinline__ void radix_digit(const uint32_t* hist, uint32_t* bcast, int shift, uint32_t dmask,
                                            uint32_t& prefix, uint32_t& pmask, uint32_t& krem) {
    if (threadIdx.x < WAVE) {
        // lane l holds bins 4l..4l+3; suffix sums from the top bin down
        const int l = lane_id();
        const uint32_t h0 = hist[4 * l], h1 = hist[4 * l + 1], h2 = hist[4 * l + 2], h3 = hist[4 * l + 3];
        uint32_t su = h0 + h1 + h2 + h3;
#pragma unroll
        for (int o = 1; o < WAVE; o <<= 1) {
            const uint32_t t = (uint32_t)__shfl_down((int)su, o, WAVE);
            if (l + o < WAVE) su += t;
        }
        // su = sum of bins >= 4l; suffix(d) for this lane's bins:
        const uint32_t s3 = su - h0 - h1 - h2, s2 = s3 + h2, s1 = s2 + h1, s0 = s1 + h0;
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
    __syncthreads();  // bcast and hist are rewritten in the next pass
}

template <int T, int EPT, bool EF, class Src>
__global__ void __launch_bounds__(T)
k_enc_topk(Src src, float* __restrict__ ef, int64_t n, int64_t nb, int32_t k, float* __restrict__ values,
           uint32_t* __restrict__ indices) {
    constexpr int B = T * EPT;
    constexpr int NW = T / WAVE;
    constexpr int CAPW = 32;               // candidates one wave may hand over
    constexpr int QC = (NW * CAPW + WAVE - 1) / WAVE;  // candidates per lane of wave 0
    __shared__ uint32_t hist[256];
    __shared__ uint32_t bcast[4];
    __shared__ uint32_t scan_lds[2 * NW];
    __shared__ uint32_t cbits[NW * CAPW];  // candidates of wave w at [w*CAPW, ...): fp32 bits,
    __shared__ uint32_t cidx[NW * CAPW];   // index in the bucket,
    __shared__ uint32_t csel[NW * CAPW];   // and whether it is sent
    __shared__ uint32_t wcount[NW];

    for (int64_t bk = blockIdx.x; bk < nb; bk += gridDim.x) {
        const int64_t lo = bk * B;
        const int64_t cnt = n - lo < B ? n - lo : B;
        const bool full = cnt == B;
        const uint32_t kb = (uint32_t)((int64_t)k < cnt ? k : cnt);
        const int32_t first = threadIdx.x * EPT;  // local index of this thread's element 0

        // a thread's EPT elements are 4*EPT contiguous bytes; plain stores
        // let L2 merge the lanes' pieces into whole lines
        src.prepare(lo, lo + cnt);
        float v[EPT];
        load_elems<EPT, EF>(src, ef, lo + first, n, full, v);

        const bool all = kb == (uint32_t)cnt;
        bool fast = !all && kb <= (uint32_t)KSMALL;  // block-uniform
        uint32_t my_off = 0, tw = 0;                 // this thread's first candidate slot; its wave's bound
        if (fast) {
            // The wave's bound tw: the kb-th largest of its threads' maxima.
            // kb elements of the bucket are at or above it, so the bucket's
            // threshold is too, and elements below tw are never sent.
            uint32_t lmax = 0;
#pragma unroll
            for (int e = 0; e < EPT; ++e)
                if (first + e < cnt) {
                    const uint32_t k1 = mag_key(v[e]) + 1u;
                    lmax = k1 > lmax ? k1 : lmax;
                }
            uint32_t c1[1] = {lmax};
            const uint32_t tw1 = wave_rth_largest<1>(c1, kb);
            tw = tw1 == 0 ? 0u : tw1 - 1u;
            uint32_t nc = 0;
#pragma unroll
            for (int e = 0; e < EPT; ++e) nc += (first + e < cnt && mag_key(v[e]) >= tw) ? 1u : 0u;
            uint32_t wtotal;
            my_off = wave_excl_scan(nc, wtotal);
            if (wtotal <= (uint32_t)CAPW) {
                uint32_t o = wave_id() * CAPW + my_off;
#pragma unroll
                for (int e = 0; e < EPT; ++e)
                    if (first + e < cnt && mag_key(v[e]) >= tw) {
                        cbits[o] = __float_as_uint(v[e]);
                        cidx[o] = (uint32_t)(first + e);
                        ++o;
                    }
            }
            if (lane_id() == 0) wcount[wave_id()] = wtotal;
            __syncthreads();
            uint32_t total = 0;
            bool over = false;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                over = over || wcount[w] > (uint32_t)CAPW;
                total += wcount[w];
            }
            fast = !over;
            if (fast && threadIdx.x < WAVE) {
                // wave 0: lane l takes candidates [l*QC, (l+1)*QC) of the
                // waves' lists one after the other, which is index order
                uint32_t pw[NW];
                uint32_t acc = 0;
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    pw[w] = acc;
                    acc += wcount[w];
                }
                uint32_t key1[QC], work[QC], slot[QC];
#pragma unroll
                for (int q = 0; q < QC; ++q) {
                    const uint32_t j = lane_id() * QC + q;
                    uint32_t sl = 0, kv = 0;
                    if (j < total) {
#pragma unroll
                        for (int w = 0; w < NW; ++w)
                            if (j >= pw[w] && j < pw[w] + wcount[w]) sl = w * CAPW + (j - pw[w]);
                        kv = (cbits[sl] & 0x7FFFFFFFu) + 1u;
                    }
                    key1[q] = work[q] = kv;
                    slot[q] = sl;
                }
                const uint32_t t1 = wave_rth_largest<QC>(work, kb);  // threshold key + 1
                uint32_t gt = 0, eq = 0;
#pragma unroll
                for (int q = 0; q < QC; ++q) {
                    gt += key1[q] > t1 ? 1u : 0u;
                    eq += key1[q] == t1 ? 1u : 0u;
                }
                uint32_t gt_all, eq_all;
                (void)wave_excl_scan(gt, gt_all);
                uint32_t eq_r = wave_excl_scan(eq, eq_all);
                const uint32_t need = kb - gt_all;
                bool sel[QC];
                uint32_t ns = 0;
#pragma unroll
                for (int q = 0; q < QC; ++q) {
                    sel[q] = key1[q] > t1;
                    if (key1[q] == t1) {
                        sel[q] = eq_r < need;
                        ++eq_r;
                    }
                    ns += sel[q] ? 1u : 0u;
                }
                uint32_t ns_all;
                uint32_t pos = wave_excl_scan(ns, ns_all);
#pragma unroll
                for (int q = 0; q < QC; ++q) {
                    const uint32_t j = lane_id() * QC + q;
                    if (j < total) csel[slot[q]] = sel[q] ? 1u : 0u;
                    if (sel[q]) {
                        values[bk * k + pos] = __uint_as_float(cbits[slot[q]]);
                        indices[bk * k + pos] = cidx[slot[q]];
                        ++pos;
                    }
                }
            }
            if (fast) __syncthreads();  // csel is visible to every thread
        }

        if (fast) {
            // the residual: sent candidates leave v - v, the rest v
            uint32_t o = wave_id() * CAPW + my_off;
#pragma unroll
            for (int q = 0; q < (EPT + 3) / 4; ++q) {
                float eo[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int e = 4 * q + j;
                    if (e >= EPT) break;
                    bool s = false;
                    if (first + e < cnt && mag_key(v[e]) >= tw) s = csel[o++] != 0u;
                    eo[j] = s ? v[e] - v[e] : v[e];
                }
                if constexpr (EF) {
                    if (EPT % 4 == 0 && full) {
                        *reinterpret_cast<f32x4*>(ef + lo + first + 4 * q) = f32x4{eo[0], eo[1], eo[2], eo[3]};
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int e = 4 * q + j;
                            if (e < EPT && first + e < cnt) ef[lo + first + e] = eo[j];
                        }
                    }
                }
            }
        } else {
            // threshold key and how many elements equal to it are still needed
            uint32_t thr = 0, need_eq = kb;
            if (!all) {
                // radix select, most significant digit first
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
                    radix_digit<T>(hist, bcast, shift, dmask, prefix, pmask, krem);
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
            uint32_t gt_r, eq_r, gt_all, eq_all;
            block_exclusive_scan2<T>(gt, eq, gt_r, eq_r, gt_all, eq_all, scan_lds);

            // pairs in index order; the residual written four elements at a time
#pragma unroll
            for (int q = 0; q < (EPT + 3) / 4; ++q) {
                float eo[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int e = 4 * q + j;
                    if (e >= EPT) break;
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
                    eo[j] = sel ? v[e] - v[e] : v[e];
                }
                if constexpr (EF) {
                    if (EPT % 4 == 0 && full) {
                        *reinterpret_cast<f32x4*>(ef + lo + first + 4 * q) = f32x4{eo[0], eo[1], eo[2], eo[3]};
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int e = 4 * q + j;
                            if (e < EPT && first + e < cnt) ef[lo + first + e] = eo[j];
                        }
                    }
                }
            }
        }
        for (int64_t j = (int64_t)kb + threadIdx.x; j < k; j += T) {
            values[bk * k + j] = 0.0f;
            indices[bk * k + j] = kNoIndex;
        }
        __syncthreads();  // LDS is reused by the next bucket
    }
}

// Buckets of 16,384 to 65,536 elements (EPT = 16 to 64 per thread of a
// 1,024-thread block).  At that block size a lane has 128 registers, too
// few to hold the thread's values, so every step reads them again in
// pieces of 16: the four radix passes, the counting pass and the emitting
// pass (the re-reads of a bucket's 64 to 256 KiB of ef and x come from L2 or
// the last-level cache).  Selection and output are those of the radix path
// above: larger keys, then equal keys by index, pairs in index order.
constexpr int TBIG = 1024;

// The index passed through an empty asm statement (no instruction): the
// compiler cannot tell that two passes read the same addresses, so it does
// not keep one pass's values in registers for the next (with one piece per
// thread it did, and spilled).
__device__ __forceinline__ int64_t fresh(int64_t i) {
    asm volatile("" : "+v"(i));
    return i;
}

template <int EPT, bool EF, class Src>
__global__ void __launch_bounds__(TBIG)
k_enc_topk_big(Src src, float* __restrict__ ef, int64_t n, int64_t nb, int32_t k, float* __restrict__ values,
               uint32_t* __restrict__ indices) {
    // pieces of 16 values (8 for 16 per thread: with the thread's values in
    // one piece the compiler kept them across passes and spilled)
    constexpr int T = TBIG, B = T * EPT, PIECE = EPT > 16 ? 16 : 8, NP = EPT / PIECE;
    static_assert(EPT % PIECE == 0, "whole pieces");
    __shared__ uint32_t hist[256];
    __shared__ uint32_t bcast[4];
    __shared__ uint32_t scan_lds[2 * (T / WAVE)];

    for (int64_t bk = blockIdx.x; bk < nb; bk += gridDim.x) {
        const int64_t lo = bk * B;
        const int64_t cnt = n - lo < B ? n - lo : B;
        const bool full = cnt == B;
        const uint32_t kb = (uint32_t)((int64_t)k < cnt ? k : cnt);
        const int32_t first = threadIdx.x * EPT;
        src.prepare(lo, lo + cnt);
        const bool all = kb == (uint32_t)cnt;

        uint32_t thr = 0, need_eq = kb;
        if (!all) {
            uint32_t prefix = 0, pmask = 0, krem = kb;
#pragma unroll 1
            for (int pass = 0; pass < 4; ++pass) {
                const int shift = pass == 3 ? 0 : 23 - 8 * pass;
                const uint32_t dmask = pass == 3 ? 0x7Fu : 0xFFu;
                for (int i = threadIdx.x; i < 256; i += T) hist[i] = 0u;
                __syncthreads();
#pragma unroll 1
                for (int p = 0; p < NP; ++p) {
                    float v[PIECE];
                    load_elems<PIECE, EF>(src, ef, fresh(lo + first + p * PIECE), n, full, v);
#pragma unroll
                    for (int e = 0; e < PIECE; ++e) {
                        const uint32_t key = mag_key(v[e]);
                        if (first + p * PIECE + e < cnt && (key & pmask) == prefix)
                            atomicAdd(&hist[(key >> shift) & dmask], 1u);
                    }
                }
                __syncthreads();
                radix_digit<T>(hist, bcast, shift, dmask, prefix, pmask, krem);
            }
            thr = prefix;
            need_eq = krem;
        }

        // counts of larger and equal keys in this thread, scanned over the block
        uint32_t gt = 0, eq = 0;
#pragma unroll 1
        for (int p = 0; p < NP; ++p) {
            float v[PIECE];
            load_elems<PIECE, EF>(src, ef, fresh(lo + first + p * PIECE), n, full, v);
#pragma unroll
            for (int e = 0; e < PIECE; ++e) {
                const uint32_t key = mag_key(v[e]);
                if (first + p * PIECE + e < cnt) {
                    gt += (!all && key > thr) ? 1u : 0u;
                    eq += (all || key == thr) ? 1u : 0u;
                }
            }
        }
        uint32_t gt_r, eq_r, gt_all, eq_all;
        block_exclusive_scan2<T>(gt, eq, gt_r, eq_r, gt_all, eq_all, scan_lds);

        // pairs in index order; the residual written four elements at a time
        // (each thread rewrites only the elements it has just read)
#pragma unroll 1
        for (int p = 0; p < NP; ++p) {
            float v[PIECE];
            const int32_t f0 = first + p * PIECE;
            load_elems<PIECE, EF>(src, ef, lo + f0, n, full, v);
#pragma unroll
            for (int q = 0; q < PIECE / 4; ++q) {
                float eo[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int e = 4 * q + j;
                    const uint32_t key = mag_key(v[e]);
                    bool sel = false;
                    uint32_t pos = 0;
                    if (f0 + e < cnt) {
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
                        indices[bk * k + pos] = (uint32_t)(f0 + e);
                    }
                    eo[j] = sel ? v[e] - v[e] : v[e];
                }
                if constexpr (EF) {
                    if (full) {
                        *reinterpret_cast<f32x4*>(ef + lo + f0 + 4 * q) = f32x4{eo[0], eo[1], eo[2], eo[3]};
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (f0 + 4 * q + j < cnt) ef[lo + f0 + 4 * q + j] = eo[j];
                    }
                }
            }
        }
        for (int64_t j = (int64_t)kb + threadIdx.x; j < k; j += T) {
            values[bk * k + j] = 0.0f;
            indices[bk * k + j] = kNoIndex;
        }
        __syncthreads();  // LDS is reused by the next bucket
    }
}

constexpr int TD = 256;  // threads of the decode kernel and of the sum for k >= 64

// The bucket's span [lo, lo + cnt) of a dense vector, from/to the block's
// 16-byte aligned LDS slice (zeros, or the caller's values), by the NT
// threads of the block, 16 bytes at a time; dst + lo and src + lo are
// 16-byte aligned (buckets are multiples of 64).
template <int NT>
__device__ __forceinline__ void slice_init(const float* __restrict__ src, int64_t lo, int64_t cnt, float* slice,
                                           bool load) {
    const int64_t q4 = cnt >> 2;
    f32x4* s4 = reinterpret_cast<f32x4*>(slice);
    if (load) {
        int64_t q = threadIdx.x;
        for (; q + 3 * NT < q4; q += 4 * NT) {  // four loads in flight
            const f32x4 a = ld_f4(src + lo + 4 * q), b = ld_f4(src + lo + 4 * (q + NT)),
                        c = ld_f4(src + lo + 4 * (q + 2 * NT)), d = ld_f4(src + lo + 4 * (q + 3 * NT));
            s4[q] = a;
            s4[q + NT] = b;
            s4[q + 2 * NT] = c;
            s4[q + 3 * NT] = d;
        }
        for (; q < q4; q += NT) s4[q] = ld_f4(src + lo + 4 * q);
        for (int64_t i = 4 * q4 + threadIdx.x; i < cnt; i += NT) slice[i] = src[lo + i];
    } else {
        for (int64_t q = threadIdx.x; q < q4; q += NT) s4[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int64_t i = 4 * q4 + threadIdx.x; i < cnt; i += NT) slice[i] = 0.0f;
    }
}
template <int NT>
__device__ __forceinline__ void slice_store(float* __restrict__ dst, int64_t lo, int64_t cnt, const float* slice) {
    const int64_t q4 = cnt >> 2;
    const f32x4* s4 = reinterpret_cast<const f32x4*>(slice);
    for (int64_t q = threadIdx.x; q < q4; q += NT) *reinterpret_cast<f32x4*>(dst + lo + 4 * q) = s4[q];
    for (int64_t i = 4 * q4 + threadIdx.x; i < cnt; i += NT) dst[lo + i] = slice[i];
}

// A tile: elements [toff, toff + tile) of bucket bk, of which cnt (0 for
// a tile past n) are in the vector.  Buckets up to TILE are one tile.
constexpr int32_t TILE = 8192;
struct Tile {
    int64_t bk, lo, cnt;
    uint32_t toff;
};
// Item `item` of the (bucket, tile) sequence, 2^tshift tiles per bucket.
__device__ __forceinline__ Tile tile_of(int64_t item, int32_t tshift, int32_t tile, int32_t bucket, int64_t n) {
    Tile t;
    t.bk = item >> tshift;
    t.toff = (uint32_t)(item & ((1 << tshift) - 1)) * (uint32_t)tile;
    t.lo = t.bk * bucket + t.toff;
    const int64_t c = n - t.lo < tile ? n - t.lo : tile;
    t.cnt = c > 0 ? c : 0;
    return t;
}

// Decode: the pairs are placed into a zeroed LDS slice of the tile, which
// then goes out with one coalesced pass.
__global__ void __launch_bounds__(TD)
k_decode_topk(const float* __restrict__ values, const uint32_t* __restrict__ indices, int64_t n, int64_t nb,
              int32_t bucket, int32_t tile, int32_t tshift, int32_t k, float* __restrict__ out) {
    extern __shared__ f32x4 lds4[];
    float* slice = reinterpret_cast<float*>(lds4);
    for (int64_t item = blockIdx.x; item < (nb << tshift); item += gridDim.x) {
        const Tile t = tile_of(item, tshift, tile, bucket, n);
        const int64_t bk = t.bk, lo = t.lo, cnt = t.cnt;
        slice_init<TD>(nullptr, lo, cnt, slice, false);
        __syncthreads();
        for (int64_t j = threadIdx.x; j < k; j += TD) {
            const uint32_t r = indices[bk * k + j] - t.toff;  // wraps past any valid slot below the tile
            if ((int64_t)r < cnt) slice[r] = values[bk * k + j];
        }
        __syncthreads();
        slice_store<TD>(out, lo, cnt, slice);
        __syncthreads();
    }
}

// The sum for k >= 64: the bucket's accumulator span lives in LDS; every
// thread adds pairs of worker w, with a barrier between workers.  Pairs of
// one worker within a bucket must have distinct indices (as the encoder
// writes them).
__global__ void __launch_bounds__(TD)
k_topk_accumulate(const float* __restrict__ values, const uint32_t* __restrict__ indices, int32_t m, int64_t n,
                  int64_t nb, int32_t bucket, int32_t tile, int32_t tshift, int32_t k, float* __restrict__ acc,
                  int32_t accumulate) {
    extern __shared__ f32x4 lds4[];
    float* slice = reinterpret_cast<float*>(lds4);
    for (int64_t item = blockIdx.x; item < (nb << tshift); item += gridDim.x) {
        const Tile t = tile_of(item, tshift, tile, bucket, n);
        const int64_t bk = t.bk, lo = t.lo, cnt = t.cnt;
        slice_init<TD>(acc, lo, cnt, slice, accumulate != 0);
        __syncthreads();
        for (int32_t w = 0; w < m; ++w) {
            const int64_t base = ((int64_t)w * nb + bk) * k;
            for (int64_t j = threadIdx.x; j < k; j += TD) {
                const uint32_t r = indices[base + j] - t.toff;
                if ((int64_t)r < cnt) slice[r] = slice[r] + values[base + j];
            }
            __syncthreads();  // worker w's additions land before worker w + 1's
        }
        slice_store<TD>(acc, lo, cnt, slice);
        __syncthreads();
    }
}

// The sum for k < 64: one wave per bucket, its accumulator span in LDS.  The
// wave takes the bucket's m*k pairs in chunks of SUM_CHUNK (worker-major
// order, SUM_R per lane) and applies a chunk in sub-steps: every pending
// pair raises its owner tag (a hash of its index) to (step << 8) | (255 -
// its worker's rank in the chunk); the pairs holding the tag's value, i.e.
// the lowest pending worker among those that share the tag, add their value
// and leave.  The winners of a sub-step belong to one worker per tag, so
// their indices are distinct and they add in parallel; for any one index
// the additions happen in worker order, one sub-step after another.  A
// wave's LDS instructions are carried out in program order, so each
// sub-step sees the previous one's sums.  The number of sub-steps is the
// largest number of workers sharing a tag; when that is large (workers
// that chose the same indices) the protocol stops after a few sub-steps and
// the rest of the chunk is applied one worker at a time.  The grid holds as
// many one-wave blocks as fit at once, each working through its XCD's
// share of the buckets with the next chunk's pairs in flight while one is
// applied; neighbouring buckets run on the same XCD at about the same time,
// since the 16-byte pieces of a worker's pairs for neighbouring buckets
// share cache lines.
__device__ __forceinline__ void wave_sync() {  // orders the lanes' LDS accesses before and after
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int SUM_R = 4;
constexpr int SUM_CHUNK = SUM_R * WAVE;  // 256 pairs: a chunk spans at most 256 workers
constexpr int SUM_TAGS = 1024;

// One chunk's pairs for one lane: pair p = c + r*64 + lane of the bucket,
// its worker's rank among the chunk's workers.
struct SumPairs {
    float val[SUM_R];
    uint32_t idx[SUM_R], rank[SUM_R];
};

// Every lane issues all 2*SUM_R loads (pairs past the bucket's last read
// element 0 and are dropped), so the number of loads in flight is fixed and
// the wait for one chunk's pairs leaves the next chunk's loads outstanding.
__device__ __forceinline__ void sum_fetch(const float* __restrict__ values, const uint32_t* __restrict__ indices,
                                          int64_t nb, int32_t k, uint32_t total, int64_t bk, uint32_t c,
                                          SumPairs& P) {
    const uint32_t w0 = c / (uint32_t)k, r0 = c - w0 * (uint32_t)k;
#pragma unroll
    for (int r = 0; r < SUM_R; ++r) {
        const uint32_t q = r0 + r * WAVE + lane_id();  // pair offset from worker w0's first pair
        const uint32_t dw = q / (uint32_t)k;
        const bool ok = c + r * WAVE + lane_id() < total;
        const int64_t src = ok ? ((int64_t)(w0 + dw) * nb + bk) * k + (q - dw * (uint32_t)k) : 0;
        const float v = values[src];
        const uint32_t i = indices[src];
        P.val[r] = ok ? v : 0.0f;
        P.idx[r] = ok ? i : kNoIndex;
        P.rank[r] = dw;
    }
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return ~wave_max_u32(~v); }

// Applies one chunk's pairs (held by one wave) to the slice, exactly in
// worker order per index.  Up to SUM_TAG_STEPS sub-steps of the tag
// protocol, then, for pairs still pending (many workers on the same
// indices), one worker after another: after a sub-step, the pairs still
// pending for an index all come from later workers than those applied.
constexpr int SUM_TAG_STEPS = 4;

__device__ __forceinline__ void sum_apply(const SumPairs& P, uint32_t toff, int64_t cnt, float* slice,
                                          uint32_t* tag, uint32_t& step) {
    bool pend[SUM_R];
    uint32_t li[SUM_R];  // slot in the tile (indices below the tile wrap past cnt)
    bool any = false;
#pragma unroll
    for (int r = 0; r < SUM_R; ++r) {
        li[r] = P.idx[r] - toff;
        pend[r] = (int64_t)li[r] < cnt;
        any = any || pend[r];
    }
    for (int sub = 0; sub < SUM_TAG_STEPS && __ballot(any) != 0; ++sub) {
        ++step;
        uint32_t mine[SUM_R], seen[SUM_R];
        // raising a tag by 0 leaves it as it is: every lane takes part
#pragma unroll
        for (int r = 0; r < SUM_R; ++r) {
            mine[r] = pend[r] ? (step << 8) | (255u - P.rank[r]) : 0u;
            atomicMax(&tag[li[r] & (SUM_TAGS - 1)], mine[r]);
        }
        wave_sync();
#pragma unroll
        for (int r = 0; r < SUM_R; ++r) seen[r] = tag[li[r] & (SUM_TAGS - 1)];
        bool win[SUM_R];
        float old[SUM_R];
#pragma unroll
        for (int r = 0; r < SUM_R; ++r) {
            win[r] = pend[r] && seen[r] == mine[r];
            old[r] = slice[win[r] ? li[r] : 0u];
        }
        wave_sync();
        any = false;
#pragma unroll
        for (int r = 0; r < SUM_R; ++r) {
            if (win[r]) slice[li[r]] = old[r] + P.val[r];
            pend[r] = pend[r] && !win[r];
            any = any || pend[r];
        }
        wave_sync();
    }
    if (__ballot(any) != 0) {
        uint32_t lo_rank = 0xFFFFFFFFu, hi_rank = 0u;
#pragma unroll
        for (int r = 0; r < SUM_R; ++r)
            if (pend[r]) {
                lo_rank = P.rank[r] < lo_rank ? P.rank[r] : lo_rank;
                hi_rank = P.rank[r] > hi_rank ? P.rank[r] : hi_rank;
            }
        const uint32_t t1 = wave_max_u32(hi_rank);
        // a worker's pairs have distinct indices: each step is one worker's
        for (uint32_t t = wave_min_u32(lo_rank); t <= t1; ++t) {
#pragma unroll
            for (int r = 0; r < SUM_R; ++r)
                if (pend[r] && P.rank[r] == t) slice[li[r]] = slice[li[r]] + P.val[r];
            wave_sync();
        }
    }
}

// One chunk of a tile: chunk 0 first sets up the slice and the tags, the
// tile's last chunk writes the slice out.
__device__ __forceinline__ void sum_chunk(const SumPairs& P, float* __restrict__ acc, const Tile& t,
                                          uint32_t total, int32_t accumulate, uint32_t c, float* slice,
                                          uint32_t* tag, uint32_t& step) {
    const int64_t lo = t.lo, cnt = t.cnt;
    if (c == 0) {
        slice_init<WAVE>(acc, lo, cnt, slice, accumulate != 0);
        for (int i = lane_id(); i < SUM_TAGS; i += WAVE) tag[i] = 0u;
        step = 0;
        wave_sync();
    }
    sum_apply(P, t.toff, cnt, slice, tag, step);
    if (c + SUM_CHUNK >= total) {
        slice_store<WAVE>(acc, lo, cnt, slice);
        wave_sync();  // the slice is rewritten by the next bucket
    }
}

__global__ void __launch_bounds__(WAVE)
k_topk_sum_wave(const float* __restrict__ values, const uint32_t* __restrict__ indices, int32_t m, int64_t n,
                int64_t nb, int32_t bucket, int32_t tile, int32_t tshift, int32_t k, float* __restrict__ acc,
                int32_t accumulate) {
    extern __shared__ f32x4 lds4[];
    float* slice = reinterpret_cast<float*>(lds4);
    uint32_t* tag = reinterpret_cast<uint32_t*>(slice + tile);    // tile is a multiple of 64
    const int64_t nitems = nb << tshift;                          // (bucket, tile) items
    const int64_t span = (nitems + 7) / 8;                        // items of one XCD
    const int64_t xcd = blockIdx.x & 7, stride = gridDim.x >> 3;  // gridDim.x is a multiple of 8
    const int64_t end = (xcd + 1) * span < nitems ? (xcd + 1) * span : nitems;
    const uint32_t total = (uint32_t)m * (uint32_t)k;             // pairs of a bucket, < 2^22

    // The wave's work is a stream of (tile, chunk) items; the pairs of the
    // next item are in flight while one is applied, alternating between two
    // register sets.  Past the last item the current one is fetched again,
    // unused.  bk runs over tiles; the pairs are those of the tile's bucket.
    int64_t bk = xcd * span + (blockIdx.x >> 3);
    uint32_t c = 0, step = 0;
    if (bk >= end) return;
    auto advance = [&](int64_t& b, uint32_t& ch) {
        ch += SUM_CHUNK;
        if (ch >= total) {
            ch = 0;
            b += stride;
        }
    };
    SumPairs A, B;
    sum_fetch(values, indices, nb, k, total, bk >> tshift, c, A);
    for (;;) {
        int64_t bk1 = bk;
        uint32_t c1 = c;
        advance(bk1, c1);
        const bool has1 = bk1 < end;
        sum_fetch(values, indices, nb, k, total, (has1 ? bk1 : bk) >> tshift, has1 ? c1 : c, B);
        sum_chunk(A, acc, tile_of(bk, tshift, tile, bucket, n), total, accumulate, c, slice, tag, step);
        if (!has1) break;
        int64_t bk2 = bk1;
        uint32_t c2 = c1;
        advance(bk2, c2);
        const bool has2 = bk2 < end;
        sum_fetch(values, indices, nb, k, total, (has2 ? bk2 : bk1) >> tshift, has2 ? c2 : c1, A);
        sum_chunk(B, acc, tile_of(bk1, tshift, tile, bucket, n), total, accumulate, c1, slice, tag, step);
        if (!has2) break;
        bk = bk2;
        c = c2;
    }
}

constexpr int64_t kLdsPerCu = 160 * 1024;  // LDS of one gfx950 compute unit

// Compute units of the current device, read once per device.  Only the
// grid size depends on it.
int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c <= 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
        cache[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

template <int T, int EPT, class Src>
hipError_t launch_enc(Src src, float* ef, int64_t n, int64_t nb, int32_t k, float* values, uint32_t* indices,
                      hipStream_t stream) {
    const dim3 grid((unsigned)grid_for(nb, 1)), block(T);
    if (ef)
        hipLaunchKernelGGL((k_enc_topk<T, EPT, true, Src>), grid, block, 0, stream, src, ef, n, nb, k, values,
                           indices);
    else
        hipLaunchKernelGGL((k_enc_topk<T, EPT, false, Src>), grid, block, 0, stream, src, ef, n, nb, k, values,
                           indices);
    return hipGetLastError();
}

template <int EPT, class Src>
hipError_t launch_enc_big(Src src, float* ef, int64_t n, int64_t nb, int32_t k, float* values, uint32_t* indices,
                          hipStream_t stream) {
    const dim3 grid((unsigned)grid_for(nb, 1)), block(TBIG);
    if (ef)
        hipLaunchKernelGGL((k_enc_topk_big<EPT, true, Src>), grid, block, 0, stream, src, ef, n, nb, k, values,
                           indices);
    else
        hipLaunchKernelGGL((k_enc_topk_big<EPT, false, Src>), grid, block, 0, stream, src, ef, n, nb, k, values,
                           indices);
    return hipGetLastError();
}

template <class Src>
hipError_t launch_topk_src(Src src, float* ef, int64_t n, int32_t bucket, int32_t k, float* values,
                           uint32_t* indices, hipStream_t stream) {
    const int64_t nb = (n + bucket - 1) / bucket;
    switch (bucket) {
        case 64: return launch_enc<64, 1>(src, ef, n, nb, k, values, indices, stream);
        case 128: return launch_enc<64, 2>(src, ef, n, nb, k, values, indices, stream);
        case 256: return launch_enc<64, 4>(src, ef, n, nb, k, values, indices, stream);
        case 512: return launch_enc<64, 8>(src, ef, n, nb, k, values, indices, stream);
        case 1024: return launch_enc<64, 16>(src, ef, n, nb, k, values, indices, stream);
        case 2048: return launch_enc<128, 16>(src, ef, n, nb, k, values, indices, stream);
        case 4096: return launch_enc<256, 16>(src, ef, n, nb, k, values, indices, stream);
        case 8192: return launch_enc<512, 16>(src, ef, n, nb, k, values, indices, stream);
        case 16384: return launch_enc_big<16>(src, ef, n, nb, k, values, indices, stream);
        case 32768: return launch_enc_big<32>(src, ef, n, nb, k, values, indices, stream);
        case 65536: return launch_enc_big<64>(src, ef, n, nb, k, values, indices, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_encode_topk(const float* x, float* ef, int64_t n, int32_t bucket, int32_t k, float* values,
                              uint32_t* indices, hipStream_t stream) {
    return launch_topk_src(FlatX{x}, ef, n, bucket, k, values, indices, stream);
}

hipError_t launch_encode_topk_list(const ListSrc& l, float* ef, int32_t bucket, int32_t k, float* values,
                                   uint32_t* indices, hipStream_t stream) {
    return launch_topk_src(list_f32(l), ef, l.n, bucket, k, values, indices, stream);
}

hipError_t launch_decode_topk(const float* values, const uint32_t* indices, int64_t n, int32_t bucket, int32_t k,
                              float* out, hipStream_t stream) {
    const int64_t nb = (n + bucket - 1) / bucket;
    const int32_t tile = bucket < TILE ? bucket : TILE;
    const int32_t tshift = log2_exact(bucket / tile);
    const size_t lds = (size_t)tile * sizeof(float);
    hipLaunchKernelGGL(k_decode_topk, dim3((unsigned)grid_for(nb << tshift, 1)), dim3(TD), lds, stream, values,
                       indices, n, nb, bucket, tile, tshift, k, out);
    return hipGetLastError();
}

hipError_t launch_topk_accumulate(const float* values, const uint32_t* indices, int32_t m, int64_t n,
                                  int32_t bucket, int32_t k, float* acc, bool accumulate, hipStream_t stream) {
    const int64_t nb = (n + bucket - 1) / bucket;
    const int32_t tile = bucket < TILE ? bucket : TILE;
    const int32_t tshift = log2_exact(bucket / tile);
    const int64_t items = nb << tshift;
    if (k < WAVE) {
        // as many one-wave blocks as the LDS of the CUs holds at once, each
        // taking its XCD's tiles in turn
        const size_t lds = (size_t)tile * sizeof(float) + SUM_TAGS * sizeof(uint32_t);
        const int64_t resident = (int64_t)cu_count() * (int64_t)(kLdsPerCu / lds);
        const int64_t want = items < resident ? items : resident;
        const int64_t grid = 8 * ((want + 7) / 8);
        hipLaunchKernelGGL(k_topk_sum_wave, dim3((unsigned)grid), dim3(WAVE), lds, stream, values, indices, m, n, nb,
                           bucket, tile, tshift, k, acc, accumulate ? 1 : 0);
    } else {
        const size_t lds = (size_t)tile * sizeof(float);
        hipLaunchKernelGGL(k_topk_accumulate, dim3((unsigned)grid_for(items, 1)), dim3(TD), lds, stream, values,
                           indices, m, n, nb, bucket, tile, tshift, k, acc, accumulate ? 1 : 0);
    }
    return hipGetLastError();
}

}  // namespace qc
