// sv_common.h -- device helpers shared by the libspecverify kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

constexpr int kWave = 64;

// 2^x as one v_exp_f32.  For x >= -126 this is exactly exp2f (whose library form adds a
// range test and a rescale around the same instruction, seven instructions in all); below,
// where exp2f returns a denormal, it may return 0.  Softmax weights that small vanish next to
// the maximum's weight of 1.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^e in fp64, to about 2e-14 relative, for every weight a sampling decision depends on
// (softmax sums, residual masses, CDF weights).  e = n + f with n = rint(e) and |f| <= 1/2;
// 2^f is a degree-9 polynomial, then scaled by 2^n.  e = -inf gives 0.  The polynomial is
// the Taylor series of exp(f ln 2) to degree 13 (first omitted term < 5e-18), economized
// to degree 9 by Chebyshev polynomials (Lanczos): with f = t/2, |t| <= 1, each top term
// b_k t^k is replaced by its expression through T_k(t) without the T_k term, whose size is
// at most |b_k| 2^(1-k) (the four dropped terms sum to 1.4e-14 of 2^f >= 0.7).  Two fewer
// multiply-adds per weight than the Taylor series to degree 11 (7e-15).
// (fp32 v_exp_f32 weights carry ~1e-7 relative error each, which moves a 128K-token CDF by
// ~1e-9: far more than the fp64 arithmetic of the decisions themselves.)
struct Exp2Poly {
    static constexpr int kTaylor = 13, kDeg = 9;
    double c[kDeg + 1];
    constexpr Exp2Poly() : c{}
    {
        const double ln2 = 0.6931471805599453094;
        double b[kTaylor + 1] = {};  // coefficients in t = 2 f
        double t = 1.0;
        for (int k = 0; k <= kTaylor; ++k) {
            double s = 1.0;
            for (int j = 0; j < k; ++j) s *= 0.5;
            b[k] = t * s;  // ln2^k / k! / 2^k
            t = t * ln2 / (double)(k + 1);
        }
        // Chebyshev polynomials T_0..T_kTaylor in the monomial basis (integer coefficients)
        double T[kTaylor + 1][kTaylor + 1] = {};
        T[0][0] = 1.0;
        T[1][1] = 1.0;
        for (int k = 1; k < kTaylor; ++k)
            for (int j = 0; j <= kTaylor; ++j)
                T[k + 1][j] = (j > 0 ? 2.0 * T[k][j - 1] : 0.0) - T[k - 1][j];
        for (int k = kTaylor; k > kDeg; --k) {
            const double q = b[k] / T[k][k];  // b_k t^k = q (T_k - lower terms of T_k)
            for (int j = 0; j < k; ++j) b[j] -= q * T[k][j];
            b[k] = 0.0;
        }
        double s = 1.0;
        for (int j = 0; j <= kDeg; ++j) {
            c[j] = b[j] * s;  // back to f: t^j = 2^j f^j
            s *= 2.0;
        }
    }
};
__device__ __forceinline__ double exp2_acc(double e)
{
    constexpr Exp2Poly P;
    e = fmax(e, -1100.0);  // below 2^-1074 the result is 0 (and -inf stays finite here)
    const double n = rint(e);
    const double f = e - n;  // exact
    double p = P.c[Exp2Poly::kDeg];
#pragma unroll
    for (int k = Exp2Poly::kDeg - 1; k >= 0; --k) p = fma(p, f, P.c[k]);
    return ldexp(p, (int)n);
}

// Every workspace starts with this fixed region of completion counters.  It must be zero
// when a workspace is first used; every call leaves it zero again.  Partial results live
// after it, so calls of any entry point and any shape can share one workspace (if they do
// not overlap in time) without finding stale data where a counter should be.
constexpr size_t kCounterBytes = 128 * 1024;
constexpr int kMaxCounters = (int)(kCounterBytes / sizeof(int));
constexpr uint64_t kTagAccept = 0x53560001ULL;
constexpr uint64_t kTagWalk = 0x53560002ULL;
constexpr uint64_t kTagGumbel = 0x53560003ULL;
constexpr uint64_t kTagRRS = 0x53560004ULL;

// Compute units of the current device (host side, asked of the runtime on every call:
// the library keeps no state between calls).  Looping kernels size their grids from it.
static inline int device_cu_count()
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    return n;
}

// ---------------------------------------------------------------------------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3", SC'11).  Each round multiplies counter words 0 and 2 by two fixed
// 64-bit constants (full 128-bit products), swaps the halves into the output
// words XOR-ed with the other counter words and the key, and the key advances by
// two Weyl increments.  Ten rounds.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1)
{
    const uint64_t M0 = 0xD2E7470EE14C6C93ULL, M1 = 0xCA5A826395121157ULL;
    const uint64_t W0 = 0x9E3779B97F4A7C15ULL, W1 = 0xBB67AE8584CAA73BULL;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t lo0 = M0 * c[0], hi0 = __umul64hi(M0, c[0]);
        const uint64_t lo1 = M1 * c[2], hi1 = __umul64hi(M1, c[2]);
        const uint64_t n0 = hi1 ^ c[1] ^ k0;
        const uint64_t n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
        k0 += W0;
        k1 += W1;
    }
}

// Uniform in (0,1): counter (index, step, stream, tag), key (seed, 0), first word
// mapped to (2*(w >> 12) + 1) * 2^-53 -- exact in fp64, never 0 or 1.
__device__ __forceinline__ double philox_uniform(uint64_t seed, uint64_t index, uint64_t step,
                                                 uint64_t stream, uint64_t tag)
{
    uint64_t c[4] = {index, step, stream, tag};
    philox4x64_10(c, seed, 0);
    return (double)(2 * (c[0] >> 12) + 1) * 0x1p-53;
}

// ---------------------------------------------------------------------------
// wave64 cross-lane primitives on DPP lane moves (VALU operand modifiers: no LDS round
// trip, unlike shuffles, which go through ds_bpermute).  GFX9 DPP controls: row_shr:n
// moves a value n lanes up inside each row of 16 lanes; row_bcast:15 / row_bcast:31 copy
// lane 15 of each row / lane 31 into the following rows selected by the row mask.
// Lanes without a source (or outside the row mask) receive the identity `id`.
// ---------------------------------------------------------------------------
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t id, uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_move(int id, int x)
{
    return (int)dpp_u32<CTRL, ROWS>((uint32_t)id, (uint32_t)x);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_move(float id, float x)
{
    return __uint_as_float(dpp_u32<CTRL, ROWS>(__float_as_uint(id), __float_as_uint(x)));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_move(double id, double x)
{
    const uint64_t o = (uint64_t)__double_as_longlong(id), v = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = dpp_u32<CTRL, ROWS>((uint32_t)o, (uint32_t)v);
    const uint32_t hi = dpp_u32<CTRL, ROWS>((uint32_t)(o >> 32), (uint32_t)(v >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// value of lane l (l uniform across the wave)
__device__ __forceinline__ int lane_value(int x, int l) { return __builtin_amdgcn_readlane(x, l); }
__device__ __forceinline__ float lane_value(float x, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ double lane_value(double x, int l)
{
    const uint64_t v = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive scan over the 64 lanes in lane order for an associative op with identity
// id: Hillis-Steele inside each 16-lane row, then the row totals.  The combination
// order is fixed, so the result is deterministic.
template <typename T, typename Op>
__device__ __forceinline__ T wave_scan_incl(T x, T id, Op op)
{
    x = op(x, dpp_move<kDppRowShr1, 0xf>(id, x));
    x = op(x, dpp_move<kDppRowShr2, 0xf>(id, x));
    x = op(x, dpp_move<kDppRowShr4, 0xf>(id, x));
    x = op(x, dpp_move<kDppRowShr8, 0xf>(id, x));
    x = op(x, dpp_move<kDppRowBcast15, 0xa>(id, x));
    x = op(x, dpp_move<kDppRowBcast31, 0xc>(id, x));
    return x;
}

struct OpAdd {
    template <typename T>
    __device__ T operator()(T a, T b) const { return a + b; }
};
struct OpMax {
    __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
    __device__ double operator()(double a, double b) const { return fmax(a, b); }
    __device__ int operator()(int a, int b) const { return max(a, b); }
};
struct OpMin {
    __device__ int operator()(int a, int b) const { return min(a, b); }
};

// Wave totals (every lane gets the result).
template <typename T>
__device__ __forceinline__ T wave_sum(T x)
{
    return lane_value(wave_scan_incl(x, (T)0, OpAdd()), kWave - 1);
}

template <typename T>
__device__ __forceinline__ T wave_max(T x)
{
    return lane_value(wave_scan_incl(x, (T)-INFINITY, OpMax()), kWave - 1);
}

__device__ __forceinline__ int wave_max_int(int x)
{
    return lane_value(wave_scan_incl(x, (int)0x80000000, OpMax()), kWave - 1);
}

__device__ __forceinline__ int wave_min_int(int x)
{
    return lane_value(wave_scan_incl(x, 0x7fffffff, OpMin()), kWave - 1);
}

// Totals of aligned lane groups of GROUP = 16, 32 or 64 lanes (every lane gets its own
// group's total).
template <int GROUP, typename T, typename Op>
__device__ __forceinline__ T group_total(T x, T id, Op op)
{
    static_assert(GROUP == 16 || GROUP == 32 || GROUP == 64, "lane group");
    x = op(x, dpp_move<kDppRowShr1, 0xf>(id, x));
    x = op(x, dpp_move<kDppRowShr2, 0xf>(id, x));
    x = op(x, dpp_move<kDppRowShr4, 0xf>(id, x));
    x = op(x, dpp_move<kDppRowShr8, 0xf>(id, x));
    if (GROUP >= 32) x = op(x, dpp_move<kDppRowBcast15, 0xa>(id, x));
    if (GROUP == 64) x = op(x, dpp_move<kDppRowBcast31, 0xc>(id, x));
    const int g = (int)(threadIdx.x % kWave) / GROUP;
    T r = lane_value(x, GROUP - 1);
#pragma unroll
    for (int k = 1; k < kWave / GROUP; ++k) {
        const T t = lane_value(x, (k + 1) * GROUP - 1);
        if (g == k) r = t;
    }
    return r;
}

// (value, index) with the larger value winning and ties going to the lower index.
__device__ __forceinline__ void argmax_merge(float &v, int &i, float v2, int i2)
{
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}

template <int CTRL, int ROWS>
__device__ __forceinline__ void argmax_step(float &v, int &i)
{
    const float v2 = dpp_move<CTRL, ROWS>(-INFINITY, v);
    const int i2 = dpp_move<CTRL, ROWS>(0x7fffffff, i);
    argmax_merge(v, i, v2, i2);
}

__device__ __forceinline__ void wave_argmax(float &v, int &i)
{
    argmax_step<kDppRowShr1, 0xf>(v, i);
    argmax_step<kDppRowShr2, 0xf>(v, i);
    argmax_step<kDppRowShr4, 0xf>(v, i);
    argmax_step<kDppRowShr8, 0xf>(v, i);
    argmax_step<kDppRowBcast15, 0xa>(v, i);
    argmax_step<kDppRowBcast31, 0xc>(v, i);
    v = lane_value(v, kWave - 1);
    i = lane_value(i, kWave - 1);
}

// ---------------------------------------------------------------------------
// bf16 <-> fp32 (raw 16-bit patterns; round to nearest even on the way down)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h)
{
    return __uint_as_float((uint32_t)h << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)0x7fc0;  // NaN stays NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Cross-block hand-off inside one kernel ("last block done").
//
// The L2 caches of the eight XCDs are not coherent with each other, and a device-scope
// release fence (a full L2 writeback) per block serializes across the GPU at ~0.1 us per
// block.  So the blocks that publish partial results write them with coherent stores
// (agent-scope relaxed atomic stores: written through to the memory side), wait until
// those stores are complete, and only then bump the group's counter.  The one block that
// arrives last invalidates its own stale cache lines (agent-scope acquire) before it
// reads the partials with ordinary loads.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void st_coherent(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(int *p, int v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(double *p, double v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent4(float *p, float4 v)
{
    st_coherent(p + 0, v.x);
    st_coherent(p + 1, v.y);
    st_coherent(p + 2, v.z);
    st_coherent(p + 3, v.w);
}

// Every block of a group publishes its partial with st_coherent*, then calls this;
// exactly one caller (the last) gets true and may then read every partial.  The
// counter is reset to zero for the next use.
__device__ __forceinline__ bool arrive_last(int *counter, int expected, int *lds_flag)
{
    // this wave's coherent stores are complete (vector-memory counter drained) ...
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // ... and so are every other wave's
    __syncthreads();
    if (threadIdx.x == 0) {
        const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = (old == expected - 1);
        if (last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *lds_flag = last ? 1 : 0;
    }
    __syncthreads();
    const bool last = *lds_flag != 0;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return last;
}

}  // namespace sv
