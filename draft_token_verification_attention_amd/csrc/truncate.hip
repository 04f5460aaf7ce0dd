// truncate.hip -- truncated sampling distributions: top-k, then top-p, per row of logits.
//
// Sources: "Speculative decoding" (Zero to Frontier textbook, ch. 20, section 20.5), section
// "When the target samples, keep a guess with probability p over q" (p and q are the
// distributions each model really samples from, after temperature and truncation such as
// top-p); box "The speculative sampling rule", special case "A processed target"; box "Four
// ways to lose exactness without noticing" (the q of the ratio must be the draft's own
// truncated distribution, not its logits before truncation).
//
// One workgroup per row (256, 512 or 1024 threads: fewer rows, more).  Tokens are ordered
// by (logit descending, token id ascending), i.e. by a unique 56-bit composite C = (order-
// preserving key of the logit) << 24 | (2^24 - 1 - id), descending.  Both cuts keep a prefix
// of that order, so the kept set is {C >= C*} for one threshold token C*, found by a radix
// select: LDS histograms of one digit of C at a time (11, 11, 10, 8, 8, 8 bits for counts;
// 10, 10, 10, 10, 8, 8 for masses), each walked from the top to the bin where the running
// count (top-k) or mass (top-p) reaches its target.  Levels run over the row until the
// crossing bin holds at most kCap tokens; one more pass gathers them into LDS (and writes
// every other token's output), and the remaining levels run on that list.  Top-p's first
// levels bin tokens by their weight instead (16 bins per factor of two, then 1024 sub-bins
// of each), which spreads them over many more bins than the logit's leading bits do.  LDS
// stays under 48 KB for 256 threads, so three rows run on each compute unit at once.
//
// A few rows leave most of the chip idle, so with a workspace the first level of every row
// (the row max, the first key digit's counts for top-k, the first weight level for top-p
// alone) is split over many blocks per row, which add their chunk's histogram into the row's
// histogram in the workspace.  When that level already leaves at most kCap tokens to gather,
// the gathering pass is split too: each block walks the row's histogram itself, writes its
// chunk's outputs and appends its chunk's candidates to the row's list in the workspace; the
// row's block then finishes on that list.  Otherwise the row's block goes on from the
// histogram alone.  The sums are exact integers, so the result is the same either way.
//
// Top-p weighs token x by w = 2^((l_x - M) log2(e) / T) (M the row's largest logit), in fp64
// to about 2e-14, and sums the weights as integers in units of 2^-62: every sum is exact and
// independent of the order of the LDS atomics, so the kept set is deterministic, and the cut
// is the exact one for those weights.
#include "vocab_row.h"

namespace {

using namespace sv;
typedef unsigned __int128 u128;

// Threads per block: 1024 while there are at most as many rows as compute units (a row then
// has a compute unit to itself), 512 up to twice as many (two rows per compute unit), else
// 256 (three rows per compute unit).  Measured on rows of 128256 logits, top-p 0.9: one row
// 203 -> 121 us, 256 rows 232 -> 152 us with 1024 threads against 256; 320 rows 280 us
// either way, and top-k 50 then top-p 0.9 on 320 rows 135 us with 256 threads, 164 with 1024.
// 512 threads against 256, top-p 0.9: 320 rows 290 -> 242 us, 400 rows 310 -> 264, 512 rows
// 352 -> 312 (top-k 50 then top-p 0.9: 2-3% faster).
constexpr int kTrThreadsMany = 256, kTrThreadsMid = 512, kTrThreadsFew = 1024;
constexpr int kMaxSplit = 64;             // chunks per row of the split first level
constexpr int kSplitMinV = 16384;         // shorter rows are not split
constexpr int kSplitAlign = 4096;         // chunk starts are multiples of this many tokens
constexpr int kBins = 2048;               // count histogram bins (digits of at most 11 bits)
constexpr int kMassBins = 1024;           // mass histogram bins (digits of at most 10 bits)
constexpr int kCap = 2048;                // candidates gathered into LDS
constexpr int kUnroll = 8;                // float4 loads in flight per thread
constexpr int kFixBits = 62;              // a weight w in [0, 1] is floor(w 2^62)
constexpr int kLoBits = 30;               // ... added to a bin as its high and low parts
constexpr int kLevels = 6;
constexpr int kIdBits = 24;               // token ids < 2^24
constexpr uint64_t kIdMask = (1ull << kIdBits) - 1;
constexpr float kFinePerUnit = 16384.0f;  // fine weight bins per unit of log2(weight)
constexpr int kFineBits = 20;             // fine weight bins: 2^20, over 64 units

// digits of C, top first: for counts, and for masses (whose histograms have fewer bins)
__device__ __constant__ const int kShiftC[kLevels] = {45, 34, 24, 16, 8, 0};
__device__ __constant__ const int kWidthC[kLevels] = {11, 11, 10, 8, 8, 8};
__device__ __constant__ const int kShiftM[kLevels] = {46, 36, 26, 16, 8, 0};
__device__ __constant__ const int kWidthM[kLevels] = {10, 10, 10, 10, 8, 8};
template <bool MASS> __device__ __forceinline__ int dshift(int l) { return MASS ? kShiftM[l] : kShiftC[l]; }
template <bool MASS> __device__ __forceinline__ int dwidth(int l) { return MASS ? kWidthM[l] : kWidthC[l]; }

struct TruncArgs {
    int R, V;
    double kd;     // log2(e) / T, for the top-p weights
    float kb;      // kFinePerUnit log2(e) / T, for the weight bins
    int top_k;
    float top_p;
    const int32_t *k_rows;
    const float *p_rows;
    const float *in;
    float *out;
    int32_t *kept;
    int vec;       // 16-byte aligned rows with V % 4 == 0: float4 loads and stores
    // split first level (S > 0): S chunks of `chunk` tokens per row; per row in the workspace
    int S, chunk;
    float *pmax;       // [R][kMaxSplit] chunk maxima
    uint32_t *ghc;     // [R][kBins] counts of the first key digit (top-k rows)
    uint32_t *gmc;     // [R][kMassBins] counts of the first weight level (top-p-alone rows)
    uint64_t *gmhi;    // [R][kMassBins] its masses, high parts
    uint64_t *gmlo;    // [R][kMassBins] low parts
    uint64_t *glist;   // [R][kCap] composites gathered by the split gather pass
    uint32_t *gcount;  // [R] their number
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

__device__ __forceinline__ uint64_t composite(float v, int e)
{
    return ((uint64_t)order_key(v) << kIdBits) | (kIdMask - (uint64_t)e);
}

__device__ __forceinline__ int comp_id(uint64_t c) { return (int)(kIdMask - (c & kIdMask)); }

__device__ __forceinline__ float comp_value(uint64_t c) { return key_value((uint32_t)(c >> kIdBits)); }

// floor(2^((v - M) kd) 2^62) for v <= M; 0 for v = -inf.
__device__ __forceinline__ uint64_t fix_weight(float v, float M, double kd)
{
    const double w = exp2_acc(((double)v - (double)M) * kd);
    return (uint64_t)ldexp(fmin(w, 1.0), kFixBits);
}

// Fine weight bin of v: about 16384 bins per unit of -log2(w), 2^20 - 1 for w below about
// 2^-64 (and -inf); larger v, smaller (or equal) bin.  Its top 10 bits are the first weight
// level, its low 10 bits the second.  Only its monotonicity matters (the bins split the
// order; masses come from fix_weight), so it is one fp32 product.
__device__ __forceinline__ int weight_fine(float v, float M, float kb)
{
    constexpr int kTop = (1 << kFineBits) - 1;
    const float x = (M - v) * kb;
    return x < (float)kTop ? (int)x : kTop;
}

// f(value, token) over the row: each thread takes 4 consecutive tokens of every 1024, and
// issues kUnroll 16-byte loads before using them.
template <int NT, typename F>
__device__ __forceinline__ void for_range(const float *row, int lo, int V, bool vec, F f)
{
    constexpr int kStep = 4 * NT;
    const int t4 = 4 * (int)threadIdx.x;
    if (vec) {
        int e0 = lo;
        for (; e0 + kUnroll * kStep <= V; e0 += kUnroll * kStep) {
            float4 x[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) x[u] = *reinterpret_cast<const float4 *>(row + e0 + u * kStep + t4);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int e = e0 + u * kStep + t4;
                f(x[u].x, e);
                f(x[u].y, e + 1);
                f(x[u].z, e + 2);
                f(x[u].w, e + 3);
            }
        }
        for (int e = e0 + t4; e < V; e += kStep) {
            const float4 x = *reinterpret_cast<const float4 *>(row + e);
            f(x.x, e);
            f(x.y, e + 1);
            f(x.z, e + 2);
            f(x.w, e + 3);
        }
    } else {
        for (int e0 = lo + t4; e0 < V; e0 += kStep)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (e0 + j < V) f(row[e0 + j], e0 + j);
    }
}

// (lo a multiple of 4; V the range's end)
template <int NT, typename F>
__device__ __forceinline__ void for_row(const float *row, int V, bool vec, F f)
{
    for_range<NT>(row, 0, V, vec, f);
}

// out[e] = g(in[e], e) over the row, with the loads of for_row and 16-byte stores.
template <int NT, typename G>
__device__ __forceinline__ void map_range(const float *row, float *orow, int lo, int V, bool vec, G g)
{
    constexpr int kStep = 4 * NT;
    const int t4 = 4 * (int)threadIdx.x;
    if (vec) {
        int e0 = lo;
        for (; e0 + kUnroll * kStep <= V; e0 += kUnroll * kStep) {
            float4 x[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) x[u] = *reinterpret_cast<const float4 *>(row + e0 + u * kStep + t4);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int e = e0 + u * kStep + t4;
                float4 y;
                y.x = g(x[u].x, e);
                y.y = g(x[u].y, e + 1);
                y.z = g(x[u].z, e + 2);
                y.w = g(x[u].w, e + 3);
                *reinterpret_cast<float4 *>(orow + e) = y;
            }
        }
        for (int e = e0 + t4; e < V; e += kStep) {
            const float4 x = *reinterpret_cast<const float4 *>(row + e);
            float4 y;
            y.x = g(x.x, e);
            y.y = g(x.y, e + 1);
            y.z = g(x.z, e + 2);
            y.w = g(x.w, e + 3);
            *reinterpret_cast<float4 *>(orow + e) = y;
        }
    } else {
        for (int e0 = lo + t4; e0 < V; e0 += kStep)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (e0 + j < V) orow[e0 + j] = g(row[e0 + j], e0 + j);
    }
}

template <int NT, typename G>
__device__ __forceinline__ void map_row(const float *row, float *orow, int V, bool vec, G g)
{
    map_range<NT>(row, orow, 0, V, vec, g);
}

// Inclusive scan of one value per thread over the block, in thread order (Hillis-Steele in
// LDS, exact for integers).  *total gets the block's total.
template <typename T, int NT>
__device__ __forceinline__ T block_scan(T x, T *s, T *total)
{
    const int t = threadIdx.x;
    __syncthreads();
    s[t] = x;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
        const T v = t >= off ? s[t - off] : (T)0;
        __syncthreads();
        s[t] += v;
        __syncthreads();
    }
    const T r = s[t];
    *total = s[NT - 1];
    __syncthreads();
    return r;
}

template <int NT>
struct TrShared {
    uint32_t hc[kBins];         // tokens per bin
    uint64_t hw_hi[kMassBins];  // sum of (floor(w 2^62) >> 30) per bin (top-p)
    uint64_t hw_lo[kMassBins];  // sum of the low 30 bits
    uint64_t list[kCap];        // composites of the gathered tokens
    u128 scan[NT];
    uint32_t s_bin, s_n;
    u128 s_above;               // the walked quantity of the bins before the crossing one
    uint64_t s_cnt_above;
    uint64_t s_found;
    float s_max[NT / kWave];
};

template <int NT>
__device__ __forceinline__ u128 bin_mass(const TrShared<NT> &sh, int bin)
{
    return ((u128)sh.hw_hi[bin] << kLoBits) + sh.hw_lo[bin];
}

// ceil(pp W) for 0 <= pp < 1 (pp exactly m 2^-s with m < 2^24): the top-p target.
__device__ __forceinline__ u128 mass_target(float pp, u128 W)
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

// The range of tokens a selection still has to split: those passing its filter whose fine
// weight bin agrees with wf on its top 10 bits (wl = 1) or all 20 (wl = 2), and whose
// composite agrees with `prefix` on the bits of `pmask` (the digits fixed so far, top bits
// first).  The walked quantity (count, or mass) of the tokens before the range in the order
// is `above`.
struct Range {
    int wl, wf;
    uint64_t prefix, pmask;
    int level;                 // next composite digit
    u128 above, target;
    uint64_t cnt_above;
    uint32_t n;                // tokens in the range
};

__device__ __forceinline__ int wfix(const Range &rg, int fine)
{
    return rg.wl == 2 ? fine : rg.wl == 1 ? fine >> 10 : 0;
}

__device__ __forceinline__ bool in_range(const Range &rg, uint64_t c, int fine)
{
    return wfix(rg, fine) == rg.wf && (c & rg.pmask) == rg.prefix;
}

// Before the range in the order (for tokens that pass the filter).
__device__ __forceinline__ bool before_range(const Range &rg, uint64_t c, int fine)
{
    const int w = wfix(rg, fine);
    if (w != rg.wf) return w < rg.wf;
    return (c & rg.pmask) > rg.prefix;
}

template <int NT>
__device__ __forceinline__ void clear_hist(TrShared<NT> &sh, int nb, bool mass)
{
    for (int i = threadIdx.x; i < nb; i += NT) {
        sh.hc[i] = 0;
        if (mass) {
            sh.hw_hi[i] = 0;
            sh.hw_lo[i] = 0;
        }
    }
    if (threadIdx.x == 0) {  // overwritten by the thread that holds the crossing
        sh.s_bin = 0;
        sh.s_above = 0;
        sh.s_cnt_above = 0;
    }
}

template <int NT>
__device__ __forceinline__ void add_token(TrShared<NT> &sh, int bin, bool mass, uint64_t f)
{
    atomicAdd(&sh.hc[bin], 1u);
    if (mass) {
        atomicAdd((unsigned long long *)&sh.hw_hi[bin], (unsigned long long)(f >> kLoBits));
        atomicAdd((unsigned long long *)&sh.hw_lo[bin], (unsigned long long)(f & ((1ull << kLoBits) - 1)));
    }
}

// Walk the histogram (bins nb-1 down to 0 = the order): the bin where the running quantity
// reaches the target.  Sets the range's target on the first walk, moves `above` and
// `cnt_above` past the bins before it, and returns it (rg.n = its tokens).
template <bool MASS, int NT>
__device__ __forceinline__ int walk(Range &rg, int nb, bool first, int k, float pp, TrShared<NT> &sh)
{
    const int t = threadIdx.x;
    const int G = (nb + NT - 1) / NT;   // bins per thread (threads past the bins own none)
    uint64_t c_loc = 0;
    u128 w_loc = 0;
    for (int j = 0; j < G; ++j) {
        const int bin = nb - 1 - G * t - j;
        if (bin < 0) break;
        c_loc += sh.hc[bin];
        w_loc += MASS ? bin_mass(sh, bin) : (u128)sh.hc[bin];
    }
    u128 w_tot;
    const u128 w_pre = block_scan<u128, NT>(w_loc, sh.scan, &w_tot) - w_loc;
    u128 c_tot;
    const uint64_t c_pre = MASS ? (uint64_t)(block_scan<u128, NT>(c_loc, sh.scan, &c_tot) - c_loc) : (uint64_t)w_pre;
    if (first) {
        rg.target = MASS ? mass_target(pp, w_tot) : (u128)k;
        if (rg.target < 1) rg.target = 1;   // at least one token
    }
    // what this range still has to cover (at most all of it)
    u128 need = rg.target - rg.above;
    if (need > w_tot) need = w_tot;
    if (w_pre < need && need <= w_pre + w_loc) {
        u128 c = w_pre;
        uint64_t cc = c_pre;
        for (int j = 0; j < G; ++j) {
            const int bin = nb - 1 - G * t - j;
            if (bin < 0) break;
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
    const int bin = (int)sh.s_bin;
    rg.above += sh.s_above;
    rg.cnt_above += sh.s_cnt_above;
    rg.n = sh.hc[bin];
    __syncthreads();
    return bin;
}

template <bool MASS>
__device__ __forceinline__ void fix_digit(Range &rg, int bin)
{
    const int s = dshift<MASS>(rg.level), w = dwidth<MASS>(rg.level);
    rg.prefix |= (uint64_t)bin << s;
    rg.pmask |= ((1ull << w) - 1) << s;
    ++rg.level;
}

// After the first top-k level: whether the whole top-k set is gathered (top-p follows), and
// whether what is left to gather fits the list.
__device__ __forceinline__ bool topk_all(bool use_p, const Range &rk)
{
    return use_p && rk.cnt_above + rk.n <= (uint64_t)kCap;
}

__device__ __forceinline__ bool topk_fits(bool use_p, const Range &rk)
{
    return topk_all(use_p, rk) || (!use_p && rk.n <= (uint32_t)kCap);
}

// Finish a selection on the gathered list (sh.list[0 .. sh.s_n), a superset of the range):
// composite digits until one token is left.  Returns its composite.
template <bool MASS, int NT, typename Filt>
__device__ __forceinline__ uint64_t finish_in_lds(Range &rg, bool first, int k, float pp, float M, double kd, Filt filt,
                                  TrShared<NT> &sh)
{
    const int n = min((int)sh.s_n, kCap);
    while ((first || rg.n > 1) && rg.level < kLevels) {
        const int nb = 1 << dwidth<MASS>(rg.level);
        clear_hist<NT>(sh, nb, MASS);
        __syncthreads();
        const int s = dshift<MASS>(rg.level);
        for (int i = threadIdx.x; i < n; i += NT) {
            const uint64_t c = sh.list[i];
            if (filt(c) && (c & rg.pmask) == rg.prefix)
                add_token(sh, (int)((c >> s) & (uint64_t)(nb - 1)), MASS, MASS ? fix_weight(comp_value(c), M, kd) : 0);
        }
        __syncthreads();
        fix_digit<MASS>(rg, walk<MASS, NT>(rg, nb, first, k, pp, sh));
        first = false;
        if (rg.level == kLevels) break;   // every digit fixed: rg.prefix is the token
    }
    // the one token of the range
    if (threadIdx.x == 0) sh.s_found = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) {
        const uint64_t c = sh.list[i];
        if (filt(c) && (c & rg.pmask) == rg.prefix) sh.s_found = c;
    }
    __syncthreads();
    const uint64_t found = sh.s_found;
    __syncthreads();
    return found;
}

// Largest value over the block.
template <int NT>
__device__ __forceinline__ float blk_max(float v, float *scratch)
{
    v = wave_max(v);
    __syncthreads();
    if ((threadIdx.x % kWave) == 0) scratch[threadIdx.x / kWave] = v;
    __syncthreads();
    float r = scratch[0];
#pragma unroll
    for (int i = 1; i < NT / kWave; ++i) r = fmaxf(r, scratch[i]);
    return r;
}

// ---- split first level ----
__device__ __forceinline__ void row_setting(const TruncArgs &a, int r, bool &use_k, bool &want_p)
{
    const int k = a.k_rows ? a.k_rows[r] : a.top_k;
    const float pp = a.p_rows ? a.p_rows[r] : a.top_p;
    use_k = k > 0 && k < a.V;
    want_p = pp < 1.0f;
}

// The row's histograms in the workspace start at zero.
__global__ __launch_bounds__(kTrThreadsMany) void trunc_zero_kernel(TruncArgs a)
{
    const int64_t r = blockIdx.x;
    if (threadIdx.x == 0) a.gcount[r] = 0;
    for (int i = threadIdx.x; i < kBins; i += kTrThreadsMany) a.ghc[r * kBins + i] = 0;
    for (int i = threadIdx.x; i < kMassBins; i += kTrThreadsMany) {
        a.gmc[r * kMassBins + i] = 0;
        a.gmhi[r * kMassBins + i] = 0;
        a.gmlo[r * kMassBins + i] = 0;
    }
}

// Chunk c of row r: its max (rows with top-p) and, for top-k rows, the counts of the first key
// digit, added into the row's histogram.
__global__ __launch_bounds__(kTrThreadsMany) void trunc_split_count_kernel(TruncArgs a)
{
    __shared__ uint32_t hc[kBins];
    __shared__ float smax[kTrThreadsMany / kWave];
    const int c = blockIdx.x, r = blockIdx.y;
    bool use_k, want_p;
    row_setting(a, r, use_k, want_p);
    const float *row = a.in + (int64_t)r * a.V;
    const int lo = c * a.chunk, hi = min(lo + a.chunk, a.V);
    if (use_k) {
        for (int i = threadIdx.x; i < kBins; i += kTrThreadsMany) hc[i] = 0;
        __syncthreads();
    }
    float mt = -INFINITY;
    for_range<kTrThreadsMany>(row, lo, hi, a.vec != 0, [&](float v, int e) __attribute__((always_inline)) {
        mt = fmaxf(mt, v);
        if (use_k) atomicAdd(&hc[(int)(composite(v, e) >> kShiftC[0])], 1u);
    });
    const float m = blk_max<kTrThreadsMany>(mt, smax);
    if (threadIdx.x == 0) a.pmax[(int64_t)r * kMaxSplit + c] = m;
    if (use_k) {
        __syncthreads();
        for (int i = threadIdx.x; i < kBins; i += kTrThreadsMany)
            if (hc[i]) atomicAdd(&a.ghc[(int64_t)r * kBins + i], hc[i]);
    }
}

// Chunk c of a top-p-alone row: its first weight level, added into the row's histogram.
__global__ __launch_bounds__(kTrThreadsMany) void trunc_split_mass_kernel(TruncArgs a)
{
    __shared__ uint32_t hc[kMassBins];
    __shared__ uint64_t hhi[kMassBins], hlo[kMassBins];
    __shared__ float smax[kTrThreadsMany / kWave];
    const int c = blockIdx.x, r = blockIdx.y;
    bool use_k, want_p;
    row_setting(a, r, use_k, want_p);
    if (use_k || !want_p) return;
    float mt = -INFINITY;
    for (int i = threadIdx.x; i < a.S; i += kTrThreadsMany) mt = fmaxf(mt, a.pmax[(int64_t)r * kMaxSplit + i]);
    const float M = blk_max<kTrThreadsMany>(mt, smax);
    if (M == -INFINITY) return;   // (the same in every thread)
    for (int i = threadIdx.x; i < kMassBins; i += kTrThreadsMany) {
        hc[i] = 0;
        hhi[i] = 0;
        hlo[i] = 0;
    }
    __syncthreads();
    const float *row = a.in + (int64_t)r * a.V;
    const int lo = c * a.chunk, hi = min(lo + a.chunk, a.V);
    for_range<kTrThreadsMany>(row, lo, hi, a.vec != 0, [&](float v, int) __attribute__((always_inline)) {
        const int bin = kMassBins - 1 - (weight_fine(v, M, a.kb) >> 10);
        const uint64_t f = fix_weight(v, M, a.kd);
        atomicAdd(&hc[bin], 1u);
        atomicAdd((unsigned long long *)&hhi[bin], (unsigned long long)(f >> kLoBits));
        atomicAdd((unsigned long long *)&hlo[bin], (unsigned long long)(f & ((1ull << kLoBits) - 1)));
    });
    __syncthreads();
    const int64_t o = (int64_t)r * kMassBins;
    for (int i = threadIdx.x; i < kMassBins; i += kTrThreadsMany)
        if (hc[i]) {
            atomicAdd(&a.gmc[o + i], hc[i]);
            atomicAdd((unsigned long long *)&a.gmhi[o + i], (unsigned long long)hhi[i]);
            atomicAdd((unsigned long long *)&a.gmlo[o + i], (unsigned long long)hlo[i]);
        }
}

// The row max from the chunk maxima of the split first level.
template <int NT>
__device__ __forceinline__ float split_max(const TruncArgs &a, int r, float *scratch)
{
    float mt = -INFINITY;
    for (int i = threadIdx.x; i < a.S; i += NT) mt = fmaxf(mt, a.pmax[(int64_t)r * kMaxSplit + i]);
    return blk_max<NT>(mt, scratch);
}

// Chunk c of row r, when the first level leaves at most kCap tokens to gather: walk the
// row's first-level histogram (as the row's block will), write the chunk's outputs and append
// its candidates to the row's list (gathered in LDS first, then one global atomic reserves
// the block's slots: one counter per row would serialize thousands of atomics).
__global__ __launch_bounds__(kTrThreadsMany, 3) void trunc_split_gather_kernel(TruncArgs a)
{
    constexpr int NT = kTrThreadsMany;
    __shared__ TrShared<NT> sh;
    const int c = blockIdx.x, r = blockIdx.y, t = threadIdx.x;
    const int k = a.k_rows ? a.k_rows[r] : a.top_k;
    const float pp = a.p_rows ? a.p_rows[r] : a.top_p;
    const bool use_k = k > 0 && k < a.V, want_p = pp < 1.0f;
    if (!use_k && !want_p) return;
    const float M = want_p ? split_max<NT>(a, r, sh.s_max) : 0.0f;
    const bool use_p = want_p && M != -INFINITY;
    if (!use_k && !use_p) return;
    const float *row = a.in + (int64_t)r * a.V;
    float *orow = a.out + (int64_t)r * a.V;
    const int lo = c * a.chunk, hi = min(lo + a.chunk, a.V);
    const bool vec = a.vec != 0;
    if (t == 0) sh.s_n = 0;   // (ordered before any append by the syncs below)
    auto append = [&](uint64_t cc) {
        const uint32_t slot = atomicAdd(&sh.s_n, 1u);
        if (slot < (uint32_t)kCap) sh.list[slot] = cc;
    };
    if (use_k) {
        Range rk{0, 0, 0, 0, 0, 0, 0, 0, (uint32_t)a.V};
        clear_hist<NT>(sh, kBins, false);
        __syncthreads();
        for (int i = t; i < kBins; i += NT) sh.hc[i] = a.ghc[(int64_t)r * kBins + i];
        __syncthreads();
        fix_digit<false>(rk, walk<false, NT>(rk, kBins, true, k, 0.0f, sh));
        if (!topk_fits(use_p, rk)) return;   // (the same in every thread)
        const bool all = topk_all(use_p, rk);
        map_range<NT>(row, orow, lo, hi, vec, [&](float v, int e) __attribute__((always_inline)) {
            const uint64_t cc = composite(v, e);
            const bool take = all ? (cc & rk.pmask) >= rk.prefix : (cc & rk.pmask) == rk.prefix;
            if (take) {
                append(cc);
                return v;   // decided by the row's block
            }
            return (!use_p && (cc & rk.pmask) > rk.prefix) ? v : -INFINITY;
        });
    } else {
        Range rp{0, 0, 0, 0, 0, 0, 0, 0, 0};
        clear_hist<NT>(sh, kMassBins, true);
        __syncthreads();
        const int64_t o = (int64_t)r * kMassBins;
        for (int i = t; i < kMassBins; i += NT) {
            sh.hc[i] = a.gmc[o + i];
            sh.hw_hi[i] = a.gmhi[o + i];
            sh.hw_lo[i] = a.gmlo[o + i];
        }
        __syncthreads();
        rp.wf = kMassBins - 1 - walk<true, NT>(rp, kMassBins, true, 0, pp, sh);
        rp.wl = 1;
        if (rp.n > (uint32_t)kCap) return;
        map_range<NT>(row, orow, lo, hi, vec, [&](float v, int e) __attribute__((always_inline)) {
            const uint64_t cc = composite(v, e);
            const int wb = weight_fine(v, M, a.kb);
            if (in_range(rp, cc, wb)) {
                append(cc);
                return v;
            }
            return before_range(rp, cc, wb) ? v : -INFINITY;
        });
    }
    // the block's candidates into the row's list
    __syncthreads();
    const uint32_t n = min(sh.s_n, (uint32_t)kCap);
    if (n == 0) return;
    if (t == 0) sh.s_bin = atomicAdd(a.gcount + r, n);
    __syncthreads();
    const uint32_t base = sh.s_bin;
    uint64_t *lst = a.glist + (int64_t)r * kCap;
    for (uint32_t i = t; i < n; i += NT)
        if (base + i < (uint32_t)kCap) lst[base + i] = sh.list[i];
}

// The candidates the split gather pass listed, into the block's list.
template <int NT>
__device__ __forceinline__ void load_split_list(const TruncArgs &a, int r, TrShared<NT> &sh)
{
    const int n = (int)min(a.gcount[r], (uint32_t)kCap);
    for (int i = threadIdx.x; i < n; i += NT) sh.list[i] = a.glist[(int64_t)r * kCap + i];
    if (threadIdx.x == 0) sh.s_n = (uint32_t)n;
    __syncthreads();
}

template <int NT>
__global__ __launch_bounds__(NT, NT == kTrThreadsMany ? 3 : 4) void truncate_kernel(TruncArgs a)
{
    __shared__ TrShared<NT> sh;
    const int r = blockIdx.x;
    const int t = threadIdx.x;
    const float *row = a.in + (int64_t)r * a.V;
    float *orow = a.out + (int64_t)r * a.V;
    const int V = a.V;
    const bool vec = a.vec != 0;
    const int k = a.k_rows ? a.k_rows[r] : a.top_k;
    const float pp = a.p_rows ? a.p_rows[r] : a.top_p;
    const bool use_k = k > 0 && k < V, want_p = pp < 1.0f;

    if (!use_k && !want_p) {  // nothing to cut
        if (orow != row) map_row<NT>(row, orow, V, vec, [](float v, int) { return v; });
        if (a.kept && t == 0) a.kept[r] = V;
        return;
    }

    auto none = [](uint64_t) { return true; };
    float M = -INFINITY;
    Range rk{0, 0, 0, 0, 0, 0, 0, 0, (uint32_t)V};

    // ---- top-k: count histogram of the first digit over the row (and the row max) ----
    if (use_k) {
        clear_hist<NT>(sh, kBins, false);   // (also the walk's crossing slots)
        if (a.S) {  // the first digit's counts came from the split pass
            __syncthreads();
            for (int i = t; i < kBins; i += NT) sh.hc[i] = a.ghc[(int64_t)r * kBins + i];
            if (want_p) M = split_max<NT>(a, r, sh.s_max);
        } else {
            __syncthreads();
            float mt = -INFINITY;
            for_row<NT>(row, V, vec, [&](float v, int e) __attribute__((always_inline)) {
                if (want_p) mt = fmaxf(mt, v);
                atomicAdd(&sh.hc[(int)(composite(v, e) >> kShiftC[0])], 1u);
            });
            if (want_p) M = blk_max<NT>(mt, sh.s_max);
        }
        __syncthreads();
        fix_digit<false>(rk, walk<false, NT>(rk, kBins, true, k, 0.0f, sh));
    } else if (a.S) {
        M = split_max<NT>(a, r, sh.s_max);
    } else {
        float mt = -INFINITY;
        for_row<NT>(row, V, vec, [&](float v, int) __attribute__((always_inline)) { mt = fmaxf(mt, v); });
        M = blk_max<NT>(mt, sh.s_max);
    }
    // a row of -inf logits has no distribution to truncate: top-p leaves it as it is
    const bool use_p = want_p && M != -INFINITY;
    const double kd = a.kd;
    const float kb = a.kb;
    if (!use_k && !use_p) {
        if (orow != row) map_row<NT>(row, orow, V, vec, [](float v, int) { return v; });
        if (a.kept && t == 0) a.kept[r] = V;
        return;
    }

    uint64_t ck = 0;   // top-k threshold (use_k)
    bool lds_k = false;
    if (use_k) {
        // whole top-k set in LDS (then top-p runs there too), or only the range
        const bool all = topk_all(use_p, rk);
        // (split, and it fits: the split gather pass has written the outputs and the list)
        const bool listed = a.S && topk_fits(use_p, rk);
        while (!listed && !all && rk.n > (uint32_t)kCap && rk.level < kLevels) {  // one more digit over the row
            const int nb = 1 << dwidth<false>(rk.level);
            clear_hist<NT>(sh, nb, false);
            __syncthreads();
            const int s = dshift<false>(rk.level);
            for_row<NT>(row, V, vec, [&](float v, int e) __attribute__((always_inline)) {
                const uint64_t c = composite(v, e);
                if ((c & rk.pmask) == rk.prefix) atomicAdd(&sh.hc[(int)((c >> s) & (uint64_t)(nb - 1))], 1u);
            });
            __syncthreads();
            fix_digit<false>(rk, walk<false, NT>(rk, nb, false, k, 0.0f, sh));
        }
        // gather; when top-k is the last cut (or the whole set is gathered) also write the
        // output of every token outside the list
        if (t == 0) sh.s_n = 0;
        __syncthreads();
        const bool write = !use_p || all;
        auto gather = [&](float v, int e) __attribute__((always_inline)) {
            const uint64_t c = composite(v, e);
            const bool take = all ? (c & rk.pmask) >= rk.prefix : (c & rk.pmask) == rk.prefix;
            if (take) {
                const uint32_t slot = atomicAdd(&sh.s_n, 1u);
                if (slot < (uint32_t)kCap) sh.list[slot] = c;
                return v;   // decided after the selection
            }
            return (!use_p && (c & rk.pmask) > rk.prefix) ? v : -INFINITY;
        };
        if (listed)
            load_split_list<NT>(a, r, sh);
        else if (write)
            map_row<NT>(row, orow, V, vec, gather);
        else
            for_row<NT>(row, V, vec, [&](float v, int e) __attribute__((always_inline)) { (void)gather(v, e); });
        __syncthreads();
        ck = finish_in_lds<false, NT>(rk, false, k, 0.0f, 0.0f, 0.0, none, sh);
        lds_k = all;
    }
    auto in_k = [&](uint64_t c) { return !use_k || c >= ck; };

    uint64_t cstar = ck;
    uint64_t n_kept = use_k ? (uint64_t)k : (uint64_t)V;
    if (use_p) {
        Range rp{0, 0, 0, 0, 0, 0, 0, 0, 0};
        if (lds_k) {
            // the whole top-k set is in the list: top-p there, from the first digit
            cstar = finish_in_lds<true, NT>(rp, true, 0, pp, M, kd, in_k, sh);
        } else {
            // first level: weight bins (over the row, or from the split pass for top-p alone)
            clear_hist<NT>(sh, kMassBins, true);
            __syncthreads();
            if (a.S && !use_k) {
                const int64_t o = (int64_t)r * kMassBins;
                for (int i = t; i < kMassBins; i += NT) {
                    sh.hc[i] = a.gmc[o + i];
                    sh.hw_hi[i] = a.gmhi[o + i];
                    sh.hw_lo[i] = a.gmlo[o + i];
                }
            } else {
                for_row<NT>(row, V, vec, [&](float v, int e) __attribute__((always_inline)) {
                    if (in_k(composite(v, e)))
                        add_token(sh, kMassBins - 1 - (weight_fine(v, M, kb) >> 10), true, fix_weight(v, M, kd));
                });
            }
            __syncthreads();
            rp.wf = kMassBins - 1 - walk<true, NT>(rp, kMassBins, true, 0, pp, sh);
            rp.wl = 1;
            // (split, top-p alone, and it fits: the split gather pass has done the gathering)
            const bool listed = a.S && !use_k && rp.n <= (uint32_t)kCap;
            if (!listed && rp.n > (uint32_t)kCap) {  // second level: the weight bin's 1024 sub-bins
                clear_hist<NT>(sh, kMassBins, true);
                __syncthreads();
                for_row<NT>(row, V, vec, [&](float v, int e) __attribute__((always_inline)) {
                    const int fine = weight_fine(v, M, kb);
                    if ((fine >> 10) == rp.wf && in_k(composite(v, e)))
                        add_token(sh, kMassBins - 1 - (fine & 1023), true, fix_weight(v, M, kd));
                });
                __syncthreads();
                rp.wf = (rp.wf << 10) | (kMassBins - 1 - walk<true, NT>(rp, kMassBins, false, 0, pp, sh));
                rp.wl = 2;
            }
            while (rp.n > (uint32_t)kCap && rp.level < kLevels) {  // composite digits over the row, inside the weight bin
                const int nb = 1 << dwidth<true>(rp.level);
                clear_hist<NT>(sh, nb, true);
                __syncthreads();
                const int s = dshift<true>(rp.level);
                for_row<NT>(row, V, vec, [&](float v, int e) __attribute__((always_inline)) {
                    const uint64_t c = composite(v, e);
                    if (in_k(c) && in_range(rp, c, weight_fine(v, M, kb)))
                        add_token(sh, (int)((c >> s) & (uint64_t)(nb - 1)), true, fix_weight(v, M, kd));
                });
                __syncthreads();
                fix_digit<true>(rp, walk<true, NT>(rp, nb, false, 0, pp, sh));
            }
            // gather the range; write every other token's output
            if (listed) {
                load_split_list<NT>(a, r, sh);
            } else {
                if (t == 0) sh.s_n = 0;
                __syncthreads();
                map_row<NT>(row, orow, V, vec, [&](float v, int e) __attribute__((always_inline)) {
                    const uint64_t c = composite(v, e);
                    if (!in_k(c)) return -INFINITY;
                    const int wb = weight_fine(v, M, kb);
                    if (in_range(rp, c, wb)) {
                        const uint32_t slot = atomicAdd(&sh.s_n, 1u);
                        if (slot < (uint32_t)kCap) sh.list[slot] = c;
                        return v;   // decided after the selection
                    }
                    return before_range(rp, c, wb) ? v : -INFINITY;
                });
            }
            __syncthreads();
            // the range's remaining digits (the weight bin no longer matters inside the list)
            cstar = finish_in_lds<true, NT>(rp, false, 0, pp, M, kd, in_k, sh);
        }
        n_kept = rp.cnt_above + 1;
    }

    // the gathered tokens: kept iff C >= C*
    const int n = min((int)sh.s_n, kCap);
    for (int i = t; i < n; i += NT) {
        const uint64_t c = sh.list[i];
        const int id = comp_id(c);
        orow[id] = c >= cstar ? row[id] : -INFINITY;
    }
    if (a.kept && t == 0) a.kept[r] = (int32_t)n_kept;
}

}  // namespace

namespace {

bool trunc_ok(const sv_trunc_desc *d)
{
    if (!d || d->R < 0 || d->V < 1) return false;
    if (!(d->temperature > 0.0f) || d->temperature == INFINITY) return false;
    return d->top_p == d->top_p;  // not NaN
}

// Whether the first level runs split (few rows, long enough), and its workspace.  Measured on
// rows of 128256 logits (without -> with): top-p 0.9 alone, 1 row 121 -> 61 us, 11 rows 122 ->
// 68, 64 rows 129 -> 87, 128 rows 134 -> 113, 256 rows 151 -> 171; top-k 50 then top-p 0.9,
// 1 row 68 -> 45, 64 rows 78 -> 68, 128 rows 81 -> 84.  So up to a quarter of the compute units.
bool trunc_split(const sv_trunc_desc *d, int cus) { return d->R > 0 && 4 * d->R <= cus && d->V >= kSplitMinV; }

size_t trunc_split_bytes(const sv_trunc_desc *d)
{
    const size_t per = kBins * sizeof(uint32_t) + kMassBins * (sizeof(uint32_t) + 2 * sizeof(uint64_t)) +
                       kMaxSplit * sizeof(float) + kCap * sizeof(uint64_t) + sizeof(uint32_t);
    return kCounterBytes + (size_t)d->R * per;
}

}  // namespace

extern "C" size_t sv_truncate_workspace(const sv_trunc_desc *d)
{
    if (!trunc_ok(d) || d->V > (1 << kIdBits) || !trunc_split(d, device_cu_count())) return 0;
    return trunc_split_bytes(d);
}

extern "C" sv_status sv_truncate(const sv_trunc_desc *d, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!trunc_ok(d)) return SV_ERR_INVALID_ARG;
    if (d->V > (1 << kIdBits)) return SV_ERR_UNSUPPORTED;  // ids in 24 bits; masses below 2^86 units
    if (d->R == 0) return SV_OK;
    if (!d->logits || !d->out) return SV_ERR_INVALID_ARG;
    TruncArgs a;
    a.R = d->R;
    a.V = d->V;
    a.kd = 1.4426950408889634 / (double)d->temperature;
    a.kb = (float)(kFinePerUnit * a.kd);
    a.top_k = d->top_k;
    a.top_p = d->top_p;
    a.k_rows = d->top_k_rows;
    a.p_rows = d->top_p_rows;
    a.in = d->logits;
    a.out = d->out;
    a.kept = d->kept;
    a.vec = (d->V % 4 == 0) && (((uintptr_t)d->logits & 15) == 0) && (((uintptr_t)d->out & 15) == 0);
    a.S = 0;
    a.chunk = 0;
    a.pmax = nullptr;
    a.ghc = nullptr;
    a.gmc = nullptr;
    a.gmhi = a.gmlo = nullptr;
    a.glist = nullptr;
    a.gcount = nullptr;
    const int cus = device_cu_count();
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    if (trunc_split(d, cus) && workspace && workspace_bytes >= trunc_split_bytes(d)) {
        // about two blocks per compute unit over all rows, chunks a multiple of 4096 tokens
        const int want = min(kMaxSplit, max(1, 2 * cus / d->R));
        const int64_t chunk = ((int64_t)(d->V + want - 1) / want + kSplitAlign - 1) / kSplitAlign * kSplitAlign;
        a.chunk = (int)chunk;
        a.S = (int)((d->V + chunk - 1) / chunk);
        char *w = static_cast<char *>(workspace) + kCounterBytes;
        a.glist = reinterpret_cast<uint64_t *>(w);
        w += (size_t)d->R * kCap * sizeof(uint64_t);
        a.ghc = reinterpret_cast<uint32_t *>(w);
        w += (size_t)d->R * kBins * sizeof(uint32_t);
        a.gmhi = reinterpret_cast<uint64_t *>(w);
        w += (size_t)d->R * kMassBins * sizeof(uint64_t);
        a.gmlo = reinterpret_cast<uint64_t *>(w);
        w += (size_t)d->R * kMassBins * sizeof(uint64_t);
        a.gmc = reinterpret_cast<uint32_t *>(w);
        w += (size_t)d->R * kMassBins * sizeof(uint32_t);
        a.pmax = reinterpret_cast<float *>(w);
        w += (size_t)d->R * kMaxSplit * sizeof(float);
        a.gcount = reinterpret_cast<uint32_t *>(w);
        const dim3 g((unsigned)a.S, (unsigned)d->R);
        // top-p alone somewhere: a row without top-k (per-row values may say so) and with top-p
        const bool mass = (d->top_k_rows || d->top_k <= 0 || d->top_k >= d->V) && (d->top_p_rows || d->top_p < 1.0f);
        hipLaunchKernelGGL(trunc_zero_kernel, dim3((unsigned)d->R), dim3(kTrThreadsMany), 0, s, a);
        hipLaunchKernelGGL(trunc_split_count_kernel, g, dim3(kTrThreadsMany), 0, s, a);
        if (mass) hipLaunchKernelGGL(trunc_split_mass_kernel, g, dim3(kTrThreadsMany), 0, s, a);
        hipLaunchKernelGGL(trunc_split_gather_kernel, g, dim3(kTrThreadsMany), 0, s, a);
        hipLaunchKernelGGL(truncate_kernel<kTrThreadsFew>, dim3((unsigned)d->R), dim3(kTrThreadsFew), 0, s, a);
    } else if (d->R <= cus) {
        hipLaunchKernelGGL(truncate_kernel<kTrThreadsFew>, dim3((unsigned)d->R), dim3(kTrThreadsFew), 0, s, a);
    } else if (d->R <= 2 * cus) {
        hipLaunchKernelGGL(truncate_kernel<kTrThreadsMid>, dim3((unsigned)d->R), dim3(kTrThreadsMid), 0, s, a);
    } else {
        hipLaunchKernelGGL(truncate_kernel<kTrThreadsMany>, dim3((unsigned)d->R), dim3(kTrThreadsMany), 0, s, a);
    }
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}
