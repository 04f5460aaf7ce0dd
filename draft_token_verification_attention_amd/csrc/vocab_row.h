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

}  // namespace sv
