// qc_bucket.hpp -- how a bucket of B consecutive elements maps onto lanes.
//
// A bucket is split into W sub-buckets, one per wave, of SUB = LPB*E*K
// contiguous elements.  Inside a sub-bucket, LPB lanes each hold K chunks of
// E contiguous elements: chunk k of lane l covers elements
// [k*LPB*E + l*E, k*LPB*E + l*E + E).  Hence
//   * every load instruction of a lane group reads one contiguous span
//     (LPB*E elements), which is what HBM streaming wants;
//   * lanes l and l^1 hold adjacent chunks, so a butterfly over the group
//     pairs sibling subtrees, chunk k is the k-th contiguous LPB*E block of
//     the sub-bucket, and sub-bucket w is the w-th contiguous block of the
//     bucket: a contiguous pairwise tree is reproduced exactly by
//     (chunk-local tree) -> (butterfly over lanes) -> (tree over k) ->
//     (tree over waves).
// When W == 1 a 128-thread block holds 2 waves and each wave holds
// 64/LPB independent buckets (measured on MI355X: 2% faster than 4-wave
// blocks for the QSGD encoder, whose waves then free their slots in pairs;
// 1-wave blocks were 5% slower); when W > 1 one block of W waves holds one
// bucket and the waves combine through LDS.
#pragma once

#include "qc_device.hpp"
#include "qc_launch.hpp"

namespace qc {

template <int E_, int LPB_, int K_, int W_>
struct Geom {
    static constexpr int E = E_, LPB = LPB_, K = K_, W = W_;
    static constexpr int SUB = LPB * E * K;
    static constexpr int B = SUB * W;
    static constexpr int GROUPS = WAVE / LPB;
    static constexpr int THREADS = W > 1 ? WAVE * W : 128;
    static constexpr int BPB = W > 1 ? 1 : (THREADS / WAVE) * GROUPS;  // buckets per block
    static_assert(LPB >= 1 && LPB <= WAVE && (LPB & (LPB - 1)) == 0, "LPB");
    static_assert(W == 1 || LPB == WAVE, "multi-wave buckets use whole waves");
};

template <class G>
__device__ __forceinline__ int64_t first_bucket() {
    if constexpr (G::W > 1)
        return blockIdx.x;
    else
        return (int64_t)blockIdx.x * G::BPB + wave_id() * G::GROUPS + lane_id() / G::LPB;
}

template <class G>
__device__ __forceinline__ int64_t bucket_stride() {
    return (int64_t)gridDim.x * G::BPB;
}

// Element offset, inside its bucket, of this lane's chunk 0.
template <class G>
__device__ __forceinline__ int64_t lane_offset() {
    const int w = G::W > 1 ? wave_id() : 0;
    return (int64_t)w * G::SUB + (int64_t)(lane_id() % G::LPB) * G::E;
}

// True on exactly one lane per bucket.
template <class G>
__device__ __forceinline__ bool bucket_leader() {
    return (lane_id() % G::LPB) == 0 && (G::W == 1 || wave_id() == 0);
}

// Combine per-wave partials of a W-wave bucket through LDS (W >= 2).  The
// value must already be uniform across each wave.  lds needs W floats.
template <int W>
__device__ __forceinline__ float block_min(float v, float* lds) {
    if (lane_id() == 0) lds[wave_id()] = v;
    __syncthreads();
    float r = lds[0];
#pragma unroll
    for (int w = 1; w < W; ++w) r = fminf(r, lds[w]);
    __syncthreads();
    return r;
}

template <int W>
__device__ __forceinline__ float block_max(float v, float* lds) {
    if (lane_id() == 0) lds[wave_id()] = v;
    __syncthreads();
    float r = lds[0];
#pragma unroll
    for (int w = 1; w < W; ++w) r = fmaxf(r, lds[w]);
    __syncthreads();
    return r;
}

// Sum of per-wave subtree sums in contiguous pairwise order (wave w holds
// the w-th contiguous block).
template <int W>
__device__ __forceinline__ float block_tree_sum(float v, float* lds) {
    if (lane_id() == 0) lds[wave_id()] = v;
    __syncthreads();
    float s[W];
#pragma unroll
    for (int w = 0; w < W; ++w) s[w] = lds[w];
    __syncthreads();
    return tree_sum_regs<W>(s);
}

inline int64_t grid_for(int64_t items, int64_t per_block) {
    int64_t g = (items + per_block - 1) / per_block;
    if (g < 1) g = 1;
    return g < kMaxBlocks ? g : kMaxBlocks;
}

}  // namespace qc
