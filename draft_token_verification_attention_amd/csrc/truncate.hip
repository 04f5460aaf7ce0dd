// truncate.hip -- truncated sampling distributions: top-k, then top-p, per row of logits.
//
// Sources: "Speculative decoding" (Zero to Frontier textbook, ch. 20, section 20.5), section
// "When the target samples, keep a guess with probability p over q" (p and q are the
// distributions each model really samples from, after temperature and truncation such as
// top-p); box "The speculative sampling rule", special case "A processed target"; box "Four
// ways to lose exactness without noticing" (the q of the ratio must be the draft's own
// truncated distribution, not its logits before truncation).
//
// One block per row.  Tokens are ordered by (logit descending, token id ascending); a
// selection keeps the tokens up to a threshold (key*, id*) in that order, key an
// order-preserving 32-bit image of the logit.  key* comes from a radix select over the row
// (three passes: 11, 11 and 10 bits of the key, histograms in LDS), id* from one pass in
// token order when only some of the tokens tied at key* are kept.  Top-p weighs token x by
// w = 2^((l_x - M) log2(e) / T) (M the row's largest logit), in fp64 to about 2e-14, and sums
// the weights as integers in units of 2^-62: every sum is exact and independent of the
// order of the LDS atomics, so the kept set is deterministic, and the cut is the exact one
// for those weights.  A last pass writes the logits of kept tokens and -inf elsewhere.
#include "vocab_row.h"

namespace {

using namespace sv;
typedef unsigned __int128 u128;

constexpr int kTrThreads = kRowThreads;   // 256
constexpr int kTrBins = 2048;             // radix digits of 11, 11 and 10 bits
constexpr int kFixBits = 62;              // a weight w in [0, 1] is floor(w 2^62)
constexpr int kLoBits = 30;               // ... added to a bin as its high and low parts

struct TruncArgs {
    int R, V;
    double kd;     // log2(e) / T, for the top-p weights
    int top_k;
    float top_p;
    const int32_t *k_rows;
    const float *p_rows;
    const float *in;
    float *out;
    int32_t *kept;
    int vec;       // 16-byte aligned rows with V % 4 == 0: float4 loads
};

// Ascending with the float value (-0 taken as +0; rows hold no NaN).
__device__ __forceinline__ uint32_t order_key(float f)
{
    const uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// floor(2^((v - M) kd) 2^62) for v <= M; 0 for v = -inf.
__device__ __forceinline__ uint64_t fix_weight(float v, float M, double kd)
{
    const double w = exp2_acc(((double)v - (double)M) * kd);
    return (uint64_t)ldexp(fmin(w, 1.0), kFixBits);
}

// f(value, token) over the row; round r covers tokens [1024 r, 1024 r + 1024), thread t its
// tokens 1024 r + 4t .. 4t + 3, so a round is in token order across the threads.
template <typename F>
__device__ __forceinline__ void for_row(const float *row, int V, bool vec, F f)
{
    if (vec) {
        for (int e = 4 * (int)threadIdx.x; e < V; e += 4 * kTrThreads) {
            const float4 v = *reinterpret_cast<const float4 *>(row + e);
            f(v.x, e);
            f(v.y, e + 1);
            f(v.z, e + 2);
            f(v.w, e + 3);
        }
    } else {
        for (int e0 = 4 * (int)threadIdx.x; e0 < V; e0 += 4 * kTrThreads)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (e0 + j < V) f(row[e0 + j], e0 + j);
    }
}

// Inclusive scan of one value per thread over the block, in thread order (Hillis-Steele in
// LDS, exact for integers).  *total gets the block's total.
template <typename T>
__device__ T block_scan(T x, T *s, T *total)
{
    const int t = threadIdx.x;
    __syncthreads();
    s[t] = x;
    __syncthreads();
    for (int off = 1; off < kTrThreads; off <<= 1) {
        const T v = t >= off ? s[t - off] : (T)0;
        __syncthreads();
        s[t] += v;
        __syncthreads();
    }
    const T r = s[t];
    *total = s[kTrThreads - 1];
    __syncthreads();
    return r;
}

// A selection: of the tokens it was restricted to, those with key > key, and those with
// key == key and token <= id, are kept.
struct Sel {
    uint32_t key;
    int id;
    uint64_t n_kept;
};

struct TrShared {
    uint32_t hc[kTrBins];         // tokens per bin
    uint64_t hw_hi[kTrBins];      // sum of (floor(w 2^62) >> 30) per bin (top-p)
    uint64_t hw_lo[kTrBins];      // sum of the low 30 bits
    u128 scan[kTrThreads];
    uint32_t s_bin;
    u128 s_above;                 // the walked quantity of the bins before the crossing one
    uint64_t s_cnt_above;
    int s_id;
    uint64_t s_run;
};

__device__ __forceinline__ u128 bin_mass(const TrShared &sh, int bin)
{
    return ((u128)sh.hw_hi[bin] << kLoBits) + sh.hw_lo[bin];
}

// ceil(pp W) for 0 <= pp < 1 (pp exactly m 2^-s with m < 2^24): the top-p target.
__device__ u128 mass_target(float pp, u128 W)
{
    if (!(pp > 0.0f)) return 0;
    int e;
    const float fm = frexpf(pp, &e);               // pp = fm 2^e, fm in [0.5, 1), e <= 0
    const uint64_t m = (uint64_t)ldexpf(fm, 24);   // exact
    const int sft = 24 - e;
    const u128 P = (u128)m * W;                    // W < 2^86: no overflow
    if (sft >= 110) return P > 0 ? 1 : 0;
    return (P + (((u128)1 << sft) - 1)) >> sft;
}

// The threshold of the tokens that pass `in`, walked in the order (key descending): the key
// at which the running count reaches k (top-k), or the running mass reaches top_p times the
// mass of those tokens (top-p, MASS).  Then id* among the tokens tied at that key, in token
// order.  Every quantity is an exact integer.
template <bool MASS, typename In>
__device__ Sel radix_select(const float *row, const TruncArgs &a, float M, In in, int k, float pp, TrShared &sh)
{
    const int t = threadIdx.x;
    uint32_t prefix = 0, pmask = 0;
    uint64_t cnt_above = 0;   // tokens before the current key range
    u128 above = 0;           // the walked quantity (count or mass) before it
    u128 target = 0;
    uint32_t tie_cnt = 0;
    for (int lev = 0; lev < 3; ++lev) {
        const int shift = lev == 0 ? 21 : lev == 1 ? 10 : 0;
        const int nb = lev == 2 ? 1024 : 2048;
        for (int i = t; i < nb; i += kTrThreads) {
            sh.hc[i] = 0;
            if (MASS) {
                sh.hw_hi[i] = 0;
                sh.hw_lo[i] = 0;
            }
        }
        if (t == 0) {  // overwritten by the thread that holds the crossing
            sh.s_bin = 0;
            sh.s_above = 0;
            sh.s_cnt_above = 0;
        }
        __syncthreads();
        for_row(row, a.V, a.vec, [&](float v, int e) {
            const uint32_t key = order_key(v);
            if ((key & pmask) == prefix && in(key, e)) {
                const int bin = (int)((key >> shift) & (uint32_t)(nb - 1));
                atomicAdd(&sh.hc[bin], 1u);
                if (MASS) {
                    const uint64_t f = fix_weight(v, M, a.kd);
                    atomicAdd((unsigned long long *)&sh.hw_hi[bin], (unsigned long long)(f >> kLoBits));
                    atomicAdd((unsigned long long *)&sh.hw_lo[bin],
                              (unsigned long long)(f & ((1ull << kLoBits) - 1)));
                }
            }
        });
        __syncthreads();
        // this thread's bins, in descending key order: nb - 1 - G t - j
        const int G = nb / kTrThreads;
        uint64_t c_loc = 0;
        u128 w_loc = 0;
        for (int j = 0; j < G; ++j) {
            const int bin = nb - 1 - G * t - j;
            c_loc += sh.hc[bin];
            w_loc += MASS ? bin_mass(sh, bin) : (u128)sh.hc[bin];
        }
        u128 w_tot;
        const u128 w_pre = block_scan<u128>(w_loc, sh.scan, &w_tot) - w_loc;
        u128 c_tot128;
        const uint64_t c_pre = MASS ? (uint64_t)(block_scan<u128>(c_loc, sh.scan, &c_tot128) - c_loc)
                                    : (uint64_t)w_pre;
        if (lev == 0) {
            target = MASS ? mass_target(pp, w_tot) : (u128)k;
            if (target < 1) target = 1;   // at least one token
        }
        // what this level's tokens still have to cover (at most all of them)
        u128 need = target - above;
        if (need > w_tot) need = w_tot;
        // the thread whose bins hold the crossing, and its first bin that reaches it
        if (w_pre < need && need <= w_pre + w_loc) {
            u128 c = w_pre;
            uint64_t cc = c_pre;
            for (int j = 0; j < G; ++j) {
                const int bin = nb - 1 - G * t - j;
                const u128 w = MASS ? bin_mass(sh, bin) : (u128)sh.hc[bin];
                if (sh.hc[bin] > 0 && c + w >= need) {
                    sh.s_bin = (uint32_t)bin;
                    sh.s_above = c;
                    sh.s_cnt_above = cc;
                    break;
                }
                c += w;
                cc += sh.hc[bin];
            }
        }
        __syncthreads();
        const uint32_t bsel = sh.s_bin;
        above += sh.s_above;
        cnt_above += sh.s_cnt_above;
        prefix |= bsel << shift;
        pmask |= (uint32_t)(nb - 1) << shift;
        if (lev == 2) tie_cnt = sh.hc[bsel];
        __syncthreads();
    }
    // tokens tied at key*: keep the first `keep` of them in token order
    uint64_t keep;
    const u128 rest = target > above ? target - above : 0;
    if (MASS) {
        const uint64_t f1 = fix_weight(key_value(prefix), M, a.kd);   // every tied token's weight
        if (f1 == 0) {
            keep = tie_cnt;
        } else {  // ceil(rest / f1): an estimate, then exact corrections
            keep = (uint64_t)((double)rest / (double)f1);
            if (keep > tie_cnt) keep = tie_cnt;
            while (keep < tie_cnt && (u128)keep * f1 < rest) ++keep;
            while (keep > 1 && (u128)(keep - 1) * f1 >= rest) --keep;
        }
    } else {
        keep = (uint64_t)rest;
    }
    if (keep < 1) keep = 1;
    if (keep > tie_cnt) keep = tie_cnt;
    Sel r;
    r.key = prefix;
    r.n_kept = cnt_above + keep;
    r.id = 0x7fffffff;
    if (keep < tie_cnt) {
        // token order: rounds of 4 x 256 tokens, a block scan of each round's matches
        if (t == 0) {
            sh.s_id = -1;
            sh.s_run = 0;
        }
        __syncthreads();
        for (int e0 = 0; e0 < a.V; e0 += 4 * kTrThreads) {
            int m[4];
            uint64_t n = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = e0 + 4 * t + j;
                m[j] = 0;
                if (e < a.V) {
                    const uint32_t key = order_key(row[e]);
                    m[j] = (key == prefix && in(key, e)) ? 1 : 0;
                }
                n += m[j];
            }
            u128 tot;
            const uint64_t before = sh.s_run + (uint64_t)(block_scan<u128>(n, sh.scan, &tot) - n);
            if (before < keep && keep <= before + n) {
                uint64_t c = before;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    c += m[j];
                    if (m[j] && c == keep) sh.s_id = e0 + 4 * t + j;
                }
            }
            __syncthreads();
            if (t == 0) sh.s_run += (uint64_t)tot;
            __syncthreads();
            if (sh.s_id >= 0) break;
        }
        r.id = sh.s_id;
        __syncthreads();
    }
    return r;
}

__global__ __launch_bounds__(kTrThreads) void truncate_kernel(TruncArgs a)
{
    __shared__ TrShared sh;
    __shared__ float fscr[kTrThreads / kWave];
    const int r = blockIdx.x;
    const float *row = a.in + (int64_t)r * a.V;
    float *orow = a.out + (int64_t)r * a.V;
    const int k = a.k_rows ? a.k_rows[r] : a.top_k;
    const float pp = a.p_rows ? a.p_rows[r] : a.top_p;
    const bool use_k = k > 0 && k < a.V, want_p = pp < 1.0f;

    float mt = -INFINITY;
    if (want_p) for_row(row, a.V, a.vec, [&](float v, int) { mt = fmaxf(mt, v); });
    const float M = want_p ? block_max(mt, fscr) : 0.0f;
    // a row of -inf logits has no distribution to truncate: top-p leaves it as it is
    const bool use_p = want_p && M != -INFINITY;

    Sel sk{0u, 0x7fffffff, (uint64_t)a.V};
    if (use_k) sk = radix_select<false>(row, a, M, [](uint32_t, int) { return true; }, k, 0.0f, sh);
    auto in_k = [&](uint32_t key, int e) { return !use_k || key > sk.key || (key == sk.key && e <= sk.id); };
    Sel s = sk;
    if (use_p) s = radix_select<true>(row, a, M, in_k, 0, pp, sh);
    const bool cut = use_k || use_p;
    for_row(row, a.V, a.vec, [&](float v, int e) {
        const uint32_t key = order_key(v);
        const bool keep = !cut || (in_k(key, e) && (!use_p || key > s.key || (key == s.key && e <= s.id)));
        orow[e] = keep ? v : -INFINITY;
    });
    if (a.kept && threadIdx.x == 0) a.kept[r] = (int32_t)s.n_kept;
}

}  // namespace

extern "C" sv_status sv_truncate(const sv_trunc_desc *d, void *stream)
{
    if (!d) return SV_ERR_INVALID_ARG;
    if (d->R < 0 || d->V < 1) return SV_ERR_INVALID_ARG;
    if (!(d->temperature > 0.0f) || d->temperature == INFINITY) return SV_ERR_INVALID_ARG;
    if (d->top_p != d->top_p) return SV_ERR_INVALID_ARG;  // NaN
    if (d->V > (1 << 24)) return SV_ERR_UNSUPPORTED;  // row masses stay below 2^86 units
    if (d->R == 0) return SV_OK;
    if (!d->logits || !d->out) return SV_ERR_INVALID_ARG;
    TruncArgs a;
    a.R = d->R;
    a.V = d->V;
    a.kd = 1.4426950408889634 / (double)d->temperature;
    a.top_k = d->top_k;
    a.top_p = d->top_p;
    a.k_rows = d->top_k_rows;
    a.p_rows = d->top_p_rows;
    a.in = d->logits;
    a.out = d->out;
    a.kept = d->kept;
    a.vec = (d->V % 4 == 0) && (((uintptr_t)d->logits & 15) == 0) && (((uintptr_t)d->out & 15) == 0);
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    hipLaunchKernelGGL(truncate_kernel, dim3((unsigned)d->R), dim3(kTrThreads), 0, s, a);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}
