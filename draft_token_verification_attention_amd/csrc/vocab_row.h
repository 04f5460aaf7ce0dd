// vocab_row.h -- block-wide primitives over one chunk of an fp32 logit row
// (shared by the acceptance and tree-walk kernels).
//
// A block of kRowThreads threads owns a chunk of consecutive logits of a row.  With
// vector loads each thread reads float4 at offset 4*t + 1024*k: every wave instruction
// is one contiguous 1 KiB segment.  Positions at or beyond V read as -inf and are
// excluded from every result.
#pragma once

#include "sv_common.h"

namespace sv {

constexpr int kRowThreads = 256;

// A block owns kRowThreads * PER consecutive logits of a row (PER per thread).
template <int PER>
struct Chunk {
    static constexpr int kPer = PER;
    static constexpr int kSize = PER * kRowThreads;
};

// Index of the k-th logit a thread holds (vector layout: float4 at 4t + 1024*(k/4)).
template <bool VEC>
__device__ __forceinline__ int chunk_index(int chunk_base, int k)
{
    if (VEC) return chunk_base + 4 * (int)threadIdx.x + 1024 * (k >> 2) + (k & 3);
    return chunk_base + (int)threadIdx.x + kRowThreads * k;
}

template <bool VEC, int PER>
__device__ __forceinline__ void load_chunk(const float *__restrict__ row, int chunk_base, int V, float (&x)[PER])
{
    if (VEC) {
#pragma unroll
        for (int k4 = 0; k4 < PER / 4; ++k4) {
            const int e = chunk_base + 4 * (int)threadIdx.x + 1024 * k4;
            if (e + 3 < V) {
                const float4 f = *reinterpret_cast<const float4 *>(row + e);
                x[4 * k4 + 0] = f.x;
                x[4 * k4 + 1] = f.y;
                x[4 * k4 + 2] = f.z;
                x[4 * k4 + 3] = f.w;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) x[4 * k4 + j] = (e + j < V) ? row[e + j] : -INFINITY;
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int e = chunk_base + (int)threadIdx.x + kRowThreads * k;
            x[k] = e < V ? row[e] : -INFINITY;
        }
    }
}

// Block reductions through a small LDS scratch (one slot per wave).
__device__ __forceinline__ float block_max(float v, float *scratch)
{
    v = wave_max(v);
    const int w = threadIdx.x / kWave;
    __syncthreads();
    if ((threadIdx.x % kWave) == 0) scratch[w] = v;
    __syncthreads();
    float r = scratch[0];
#pragma unroll
    for (int i = 1; i < kRowThreads / kWave; ++i) r = fmaxf(r, scratch[i]);
    return r;
}

__device__ __forceinline__ double block_sum(double v, double *scratch)
{
    v = wave_sum(v);
    const int w = threadIdx.x / kWave;
    __syncthreads();
    if ((threadIdx.x % kWave) == 0) scratch[w] = v;
    __syncthreads();
    double r = 0.0;
#pragma unroll
    for (int i = 0; i < kRowThreads / kWave; ++i) r += scratch[i];  // fixed order: deterministic
    return r;
}

__device__ __forceinline__ void block_argmax(float &v, int &idx, float *sv, int *si)
{
    wave_argmax(v, idx);
    const int w = threadIdx.x / kWave;
    __syncthreads();
    if ((threadIdx.x % kWave) == 0) {
        sv[w] = v;
        si[w] = idx;
    }
    __syncthreads();
    v = sv[0];
    idx = si[0];
#pragma unroll
    for (int i = 1; i < kRowThreads / kWave; ++i) argmax_merge(v, idx, sv[i], si[i]);
}

__device__ __forceinline__ int block_min_int(int v, int *scratch)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
    const int w = threadIdx.x / kWave;
    __syncthreads();
    if ((threadIdx.x % kWave) == 0) scratch[w] = v;
    __syncthreads();
    int r = scratch[0];
#pragma unroll
    for (int i = 1; i < kRowThreads / kWave; ++i) r = min(r, scratch[i]);
    return r;
}

__device__ __forceinline__ int block_max_int(int v, int *scratch)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
    const int w = threadIdx.x / kWave;
    __syncthreads();
    if ((threadIdx.x % kWave) == 0) scratch[w] = v;
    __syncthreads();
    int r = scratch[0];
#pragma unroll
    for (int i = 1; i < kRowThreads / kWave; ++i) r = max(r, scratch[i]);
    return r;
}

// Exclusive prefix sum (fp64) of one value per thread, in thread order: a wave scan,
// then the wave totals (fixed order, deterministic).
__device__ __forceinline__ double block_exclusive_scan(double v, double *scratch /* >= waves */)
{
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    double incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    __syncthreads();
    if (lane == kWave - 1) scratch[w] = incl;
    __syncthreads();
    double before = 0.0;
    for (int i = 0; i < w; ++i) before += scratch[i];
    return before + incl - v;
}

// Inverse-CDF search inside one chunk, in token order, over weights w(l0[e], l1[e]) of
// one or two logit rows (l1 may be null: then w gets l0[e] twice).  `base` is the
// cumulative weight before the chunk, `target` = u * Z.  Returns the smallest e with
// base + C_e > target, or -1 when the chunk's running sum never passes it.  Two levels:
// every thread sums PER consecutive weights (16-byte loads when VEC), a block scan finds
// the segment where the running sum crosses target, and one wave scans that segment.
template <int PER, bool VEC, typename WeightFn>
__device__ __forceinline__ int chunk_inverse_cdf(const float *l0, const float *l1, int chunk_base, int V, double base,
                                                 double target, WeightFn weight, double *scratch, int *iscratch)
{
    static_assert(PER <= kWave && PER % 4 == 0, "one wave scans a segment");
    __shared__ int s_seg;
    __shared__ double s_c0;
    const int first = chunk_base + PER * (int)threadIdx.x;
    double local = 0.0;
    if (VEC && first + PER <= V) {
#pragma unroll
        for (int k4 = 0; k4 < PER / 4; ++k4) {
            const float4 a = *reinterpret_cast<const float4 *>(l0 + first + 4 * k4);
            const float4 c = l1 ? *reinterpret_cast<const float4 *>(l1 + first + 4 * k4) : a;
            local += weight(a.x, c.x) + weight(a.y, c.y) + weight(a.z, c.z) + weight(a.w, c.w);
        }
    } else {
        for (int k = 0; k < PER; ++k) {
            const int e = first + k;
            if (e < V) local += weight(l0[e], l1 ? l1[e] : l0[e]);
        }
    }
    const double c0 = base + block_exclusive_scan(local, scratch);
    const bool crossing = local > 0.0 && c0 <= target && c0 + local > target;
    const int seg = block_min_int(crossing ? (int)threadIdx.x : 0x7fffffff, iscratch);
    if (seg == 0x7fffffff) return -1;
    if ((int)threadIdx.x == seg) {
        s_seg = seg;
        s_c0 = c0;
    }
    __syncthreads();
    int found = 0x7fffffff;
    if (threadIdx.x < kWave) {
        const int lane = threadIdx.x;
        const int e = chunk_base + PER * s_seg + lane;
        const double w = (lane < PER && e < V) ? weight(l0[e], l1 ? l1[e] : l0[e]) : 0.0;
        double incl = w;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const double t = __shfl_up(incl, o);
            if (lane >= o) incl += t;
        }
        const uint64_t hit = __ballot(w > 0.0 && s_c0 + incl > target);
        const uint64_t pos = __ballot(w > 0.0);
        if (hit)
            found = chunk_base + PER * s_seg + (__ffsll((unsigned long long)hit) - 1);
        else if (pos)  // rounding: the segment's own sum stops short of target
            found = chunk_base + PER * s_seg + (63 - __clzll((unsigned long long)pos));
    }
    const int r = block_min_int(found, iscratch);
    return r == 0x7fffffff ? -1 : r;
}

// Combine per-chunk row statistics with one wave: lanes stride over the chunks.
//   max_arg: (largest value, lowest index among equals)
//   softmax: M = max m_c, Z = sum_c S_c 2^((m_c - M) k)
// Must be called by a whole wave; every lane gets the result.
template <typename Part>
__device__ __forceinline__ void wave_combine_argmax(const Part *pp, int nchunk, float &v, int &idx)
{
    const int lane = threadIdx.x % kWave;
    v = -INFINITY;
    idx = 0x7fffffff;
    for (int c = lane; c < nchunk; c += kWave) argmax_merge(v, idx, pp[c].m, pp[c].arg);
    wave_argmax(v, idx);
}

template <typename Part>
__device__ __forceinline__ void wave_combine_softmax(const Part *pp, int nchunk, double kd, float &M, double &Z)
{
    const int lane = threadIdx.x % kWave;
    float m = -INFINITY;
    for (int c = lane; c < nchunk; c += kWave) m = fmaxf(m, pp[c].m);
    M = wave_max(m);
    double z = 0.0;
    for (int c = lane; c < nchunk; c += kWave)
        if (pp[c].s > 0.0) z += pp[c].s * exp2(((double)pp[c].m - (double)M) * kd);
    // fixed-order reduction: deterministic
    Z = wave_sum(z);
}

// Find the first chunk whose running weight passes `target` (one wave; chunk weights
// come from weight(c)).  Returns the chunk and the running weight before it; when
// rounding leaves every prefix at or below target, the last chunk with weight.
template <typename WFn>
__device__ __forceinline__ void wave_find_chunk(int nchunk, double target, WFn weight, int &chunk, double &base)
{
    const int lane = threadIdx.x % kWave;
    double carry = 0.0;
    int last_pos = -1;
    double last_base = 0.0;
    chunk = -1;
    for (int c0 = 0; c0 < nchunk; c0 += kWave) {
        const int c = c0 + lane;
        const double w = c < nchunk ? weight(c) : 0.0;
        // inclusive scan across the wave (fixed order)
        double incl = w;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const double t = __shfl_up(incl, o);
            if (lane >= o) incl += t;
        }
        const double excl = carry + incl - w;
        const uint64_t pass = __ballot(c < nchunk && w > 0.0 && carry + incl > target);
        const uint64_t pos = __ballot(c < nchunk && w > 0.0);
        if (pos) {
            const int lp = 63 - __clzll((unsigned long long)pos);
            last_pos = c0 + lp;
            last_base = __shfl(excl, lp);
        }
        if (pass) {
            const int fl = __ffsll((unsigned long long)pass) - 1;
            chunk = c0 + fl;
            base = __shfl(excl, fl);
            return;
        }
        carry += __shfl(incl, kWave - 1);
    }
    chunk = last_pos < 0 ? nchunk - 1 : last_pos;
    base = last_pos < 0 ? 0.0 : last_base;
}

}  // namespace sv
