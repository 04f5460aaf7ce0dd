// vocab_row.h -- block-wide primitives over one chunk of an fp32 logit row
// (shared by the acceptance and tree-walk kernels).
//
// A block of kRowThreads threads owns kChunk consecutive logits of a row.  With
// vector loads each thread reads float4 at offset 4*t + 1024*k (k = 0..3): every
// wave instruction is one contiguous 1 KiB segment.  Positions at or beyond V
// read as -inf and are excluded from every result.
#pragma once

#include "sv_common.h"

namespace sv {

constexpr int kRowThreads = 256;
constexpr int kChunk = 4096;
constexpr int kPerThread = kChunk / kRowThreads;  // 16

// Index of the k-th logit a thread holds.
template <bool VEC>
__device__ __forceinline__ int chunk_index(int chunk_base, int k)
{
    if (VEC) return chunk_base + 4 * (int)threadIdx.x + 1024 * (k >> 2) + (k & 3);
    return chunk_base + (int)threadIdx.x + kRowThreads * k;
}

template <bool VEC>
__device__ __forceinline__ void load_chunk(const float *__restrict__ row, int chunk_base, int V, float x[kPerThread])
{
    if (VEC) {
#pragma unroll
        for (int k4 = 0; k4 < kPerThread / 4; ++k4) {
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
        for (int k = 0; k < kPerThread; ++k) {
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

// Exclusive prefix sum (fp64) of one value per thread, in thread order.
__device__ __forceinline__ double block_exclusive_scan(double v, double *scratch /* kRowThreads */)
{
    __syncthreads();
    scratch[threadIdx.x] = v;
    __syncthreads();
    // Hillis-Steele over 256 entries: fixed order, deterministic.
    for (int off = 1; off < kRowThreads; off <<= 1) {
        const double add = threadIdx.x >= (unsigned)off ? scratch[threadIdx.x - off] : 0.0;
        __syncthreads();
        scratch[threadIdx.x] += add;
        __syncthreads();
    }
    return scratch[threadIdx.x] - v;
}

// Inverse-CDF search inside one chunk of non-negative weights w(e), in token order.
// `base` is the cumulative weight before the chunk, `target` = u * Z.  Returns the
// smallest index e with base + C_e > target, or -1 when the chunk's running sum
// never passes it.  Each thread scans 16 consecutive positions.
template <typename WeightFn>
__device__ __forceinline__ int chunk_inverse_cdf(int chunk_base, int V, double base, double target,
                                                 WeightFn weight, double *scan_scratch, int *iscratch)
{
    double w[kPerThread];
    double local = 0.0;
    const int first = chunk_base + kPerThread * (int)threadIdx.x;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int e = first + k;
        w[k] = e < V ? weight(e) : 0.0;
        local += w[k];
    }
    double c = base + block_exclusive_scan(local, scan_scratch);
    int found = 0x7fffffff;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        c += w[k];
        if (found == 0x7fffffff && w[k] > 0.0 && c > target) found = first + k;
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
