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

// All of a thread's loads are issued before any is waited for, with no branch (a load
// under a branch lets the compiler wait for earlier loads at the join): vector rows read
// clamped in-bounds float4s and mask the positions at or beyond V (V % 4 == 0, so a float4
// is wholly inside or wholly beyond the row).
template <bool VEC, int PER>
__device__ __forceinline__ void load_chunk(const float *__restrict__ row, int chunk_base, int V, float (&x)[PER])
{
    if (VEC) {
        float4 f[PER / 4];
#pragma unroll
        for (int k4 = 0; k4 < PER / 4; ++k4)
            f[k4] = *reinterpret_cast<const float4 *>(row + min(chunk_base + 4 * (int)threadIdx.x + 1024 * k4, V - 4));
#pragma unroll
        for (int k4 = 0; k4 < PER / 4; ++k4) {
            const bool in = chunk_base + 4 * (int)threadIdx.x + 1024 * k4 < V;
            x[4 * k4 + 0] = in ? f[k4].x : -INFINITY;
            x[4 * k4 + 1] = in ? f[k4].y : -INFINITY;
            x[4 * k4 + 2] = in ? f[k4].z : -INFINITY;
            x[4 * k4 + 3] = in ? f[k4].w : -INFINITY;
        }
        return;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int e = chunk_index<VEC>(chunk_base, k);
        const float v = row[min(e, V - 1)];
        x[k] = e < V ? v : -INFINITY;
    }
}

// The same chunk of two rows, every load issued before any is waited for (one branch:
// full chunk or the row's last, partial chunk).
template <bool VEC, int PER>
__device__ __forceinline__ void load_chunk2(const float *__restrict__ r0, const float *__restrict__ r1, int chunk_base,
                                            int V, float (&x0)[PER], float (&x1)[PER])
{
    if (VEC) {  // clamped float4s, masked (no branch: see load_chunk)
        float4 f0[PER / 4], f1[PER / 4];
#pragma unroll
        for (int k4 = 0; k4 < PER / 4; ++k4) {
            const int e = min(chunk_base + 4 * (int)threadIdx.x + 1024 * k4, V - 4);
            f0[k4] = *reinterpret_cast<const float4 *>(r0 + e);
            f1[k4] = *reinterpret_cast<const float4 *>(r1 + e);
        }
#pragma unroll
        for (int k4 = 0; k4 < PER / 4; ++k4) {
            const bool in = chunk_base + 4 * (int)threadIdx.x + 1024 * k4 < V;
            x0[4 * k4 + 0] = in ? f0[k4].x : -INFINITY;
            x0[4 * k4 + 1] = in ? f0[k4].y : -INFINITY;
            x0[4 * k4 + 2] = in ? f0[k4].z : -INFINITY;
            x0[4 * k4 + 3] = in ? f0[k4].w : -INFINITY;
            x1[4 * k4 + 0] = in ? f1[k4].x : -INFINITY;
            x1[4 * k4 + 1] = in ? f1[k4].y : -INFINITY;
            x1[4 * k4 + 2] = in ? f1[k4].z : -INFINITY;
            x1[4 * k4 + 3] = in ? f1[k4].w : -INFINITY;
        }
        return;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int e = chunk_index<VEC>(chunk_base, k);
        const float v0 = r0[min(e, V - 1)], v1 = r1[min(e, V - 1)];
        x0[k] = e < V ? v0 : -INFINITY;
        x1[k] = e < V ? v1 : -INFINITY;
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
    v = wave_min_int(v);
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
    v = wave_max_int(v);
    const int w = threadIdx.x / kWave;
    __syncthreads();
    if ((threadIdx.x % kWave) == 0) scratch[w] = v;
    __syncthreads();
    int r = scratch[0];
#pragma unroll
    for (int i = 1; i < kRowThreads / kWave; ++i) r = max(r, scratch[i]);
    return r;
}

// Two fp64 block sums at once (one barrier pair for both).
__device__ __forceinline__ void block_sum2(double &a, double &b, double *scratch /* >= 2 * waves */)
{
    a = wave_sum(a);
    b = wave_sum(b);
    const int w = threadIdx.x / kWave;
    constexpr int NW = kRowThreads / kWave;
    __syncthreads();
    if ((threadIdx.x % kWave) == 0) {
        scratch[w] = a;
        scratch[NW + w] = b;
    }
    __syncthreads();
    a = 0.0;
    b = 0.0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {  // fixed order: deterministic
        a += scratch[i];
        b += scratch[NW + i];
    }
}

// Exclusive prefix sum (fp64) of one value per thread, in thread order: a wave scan,
// then the wave totals (fixed order, deterministic).
__device__ __forceinline__ double block_exclusive_scan(double v, double *scratch /* >= waves */)
{
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    const double incl = wave_scan_incl(v, 0.0, OpAdd());
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
// base + C_e > target; when rounding leaves the chunk's running sum at or below target,
// the last position with positive weight (-1 if none).  Every thread owns PER
// consecutive positions (16-byte loads when VEC) and sums their weights in order; a block
// scan of those sums gives each thread its running sum c0; the one thread with
// c0 <= target < c0 + its sum scans its own weights, still in registers.
template <int PER, bool VEC, typename WeightFn>
__device__ __forceinline__ int chunk_inverse_cdf(const float *l0, const float *l1, int chunk_base, int V, double base,
                                                 double target, WeightFn weight, double *scratch, int *iscratch)
{
    static_assert(PER % 4 == 0, "vector segments");
    __shared__ int s_found;
    const int first = chunk_base + PER * (int)threadIdx.x;
    const float *l1r = l1 ? l1 : l0;  // the weight ignores its second argument for one row
    double w[PER];
    if (VEC && chunk_base + PER * kRowThreads <= V) {  // full chunk: all loads issued up front
        float4 a[PER / 4], c[PER / 4];
#pragma unroll
        for (int k4 = 0; k4 < PER / 4; ++k4) {
            a[k4] = *reinterpret_cast<const float4 *>(l0 + first + 4 * k4);
            c[k4] = *reinterpret_cast<const float4 *>(l1r + first + 4 * k4);
        }
#pragma unroll
        for (int k4 = 0; k4 < PER / 4; ++k4) {
            w[4 * k4 + 0] = weight(a[k4].x, c[k4].x);
            w[4 * k4 + 1] = weight(a[k4].y, c[k4].y);
            w[4 * k4 + 2] = weight(a[k4].z, c[k4].z);
            w[4 * k4 + 3] = weight(a[k4].w, c[k4].w);
        }
    } else {
        float a[PER], c[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int e = min(first + k, V - 1);
            a[k] = l0[e];
            c[k] = l1r[e];
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) w[k] = first + k < V ? weight(a[k], c[k]) : 0.0;
    }
    double local = 0.0;
    int lastpos = -1;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        local += w[k];
        if (w[k] > 0.0) lastpos = first + k;
    }
    if (threadIdx.x == 0) s_found = 0x7fffffff;
    const double c0 = base + block_exclusive_scan(local, scratch);  // (its barriers publish s_found)
    if (c0 <= target) {
        // first own position whose running sum c0 + w_0 + ... + w_k passes target (the
        // running sum only grows where w_k > 0, so that position has mass)
        double pre = c0;
        int hit = 0x7fffffff;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            pre += w[k];
            if (hit == 0x7fffffff && pre > target) hit = first + k;
        }
        if (hit != 0x7fffffff) atomicMin(&s_found, hit);
    }
    __syncthreads();
    const int f = s_found;
    if (f != 0x7fffffff) return f;
    const int r = block_max_int(lastpos, iscratch);
    return r;
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
        if (pp[c].s > 0.0) z += pp[c].s * exp2_acc(((double)pp[c].m - (double)M) * kd);
    // fixed-order reduction: deterministic
    Z = wave_sum(z);
}

// Softmax statistics of several rows at once from their chunk partials: rows are laid
// out over aligned groups of LPR lanes (LPR = 16, 32 or 64; a lane strides over chunks
// c = lane % LPR + k LPR), so one wave pass covers 64 / LPR rows.  Per row:
// M = max_c m_c and Z = sum_c S_c 2^((m_c - M) k), the rescale factor in fp64 (exp2_acc).
// Must be called by a whole wave; `row` is this lane's row (rows >= nrows compute nothing
// useful), the results are valid in every lane of the row's group.
template <int LPR, typename Part>
__device__ __forceinline__ void group_combine_softmax(const Part *pp, int row, int nrows, int nchunk, double kd,
                                                      float &M, double &Z)
{
    const int c0 = (int)(threadIdx.x % LPR);
    float m = -INFINITY;
    if (row < nrows)
        for (int c = c0; c < nchunk; c += LPR) m = fmaxf(m, pp[(int64_t)row * nchunk + c].m);
    M = group_total<LPR>(m, -INFINITY, OpMax());
    double z = 0.0;
    if (row < nrows)
        for (int c = c0; c < nchunk; c += LPR) {
            const Part q = pp[(int64_t)row * nchunk + c];
            if (q.s > 0.0) z += q.s * exp2_acc(((double)q.m - (double)M) * kd);
        }
    Z = group_total<LPR>(z, 0.0, OpAdd());
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
        const double incl = wave_scan_incl(w, 0.0, OpAdd());
        const double excl = carry + incl - w;
        const uint64_t pass = __ballot(c < nchunk && w > 0.0 && carry + incl > target);
        const uint64_t pos = __ballot(c < nchunk && w > 0.0);
        if (pos) {
            const int lp = 63 - __clzll((unsigned long long)pos);
            last_pos = c0 + lp;
            last_base = lane_value(excl, lp);
        }
        if (pass) {
            const int fl = __ffsll((unsigned long long)pass) - 1;
            chunk = c0 + fl;
            base = lane_value(excl, fl);
            return;
        }
        carry += lane_value(incl, kWave - 1);
    }
    chunk = last_pos < 0 ? nchunk - 1 : last_pos;
    base = last_pos < 0 ? 0.0 : last_base;
}

}  // namespace sv
