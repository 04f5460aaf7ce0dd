// penalty.hip -- repetition, frequency and presence penalties on logit rows, with the drafted
// prefix as context.
//
// Sources: "Speculative decoding" (Zero to Frontier textbook, ch. 20, section 20.5), section
// "When the target samples, keep a guess with probability p over q" (p and q are the
// distributions each model really samples from, after temperature, truncation and
// penalties); box "The speculative sampling rule", special case "A processed target" (the
// target's penalties are applied with the drafted prefix as context).  The pages do not
// define the penalties; the usual three are taken: a token seen c > 0 times in the context
// has its logit l replaced by (r - c * frequency) - presence, r = l / theta if l > 0 else
// l * theta, in fp64 and rounded once to fp32.  Row i of a sequence has as context its
// history followed by its first i drafted tokens.
//
// Histories of up to kHashMaxHist entries: two launches.  One workgroup per sequence counts
// its history in an LDS hash table, writes the distinct tokens with their counts as a list,
// and looks up the history count of each drafted token.  Then one block per (sequence, chunk
// of that list) penalizes each listed token in every row of the sequence, adding row by row
// the drafts before that row; drafted tokens absent from the history are penalized by the
// sequence's first block, at their first occurrence.  Every token of a row is written by
// exactly one thread.  The call reads only what it wrote first, so it shares a workspace with
// the other entry points.
//
// Longer histories: four launches.  The first zeroes the count of every token the call will
// read (history and drafts) in a per-sequence array over the vocabulary; the second counts the
// history into it and lists the distinct tokens (the entry whose increment finds the count at
// zero appends its token; the list length lives in the counter region); the third applies as
// above; the last returns the list lengths to zero.  Work is proportional to the distinct
// tokens of the history times the rows, not to the vocabulary.
#include "sv_common.h"

namespace {

using namespace sv;

constexpr int kPenThreads = 256;
constexpr int kPenChunk = 4 * kPenThreads;   // history entries per block
constexpr int kMaxPenDrafts = 64;
constexpr int kHashThreads = 1024;
constexpr int kHashSlots = 16384;            // LDS hash table (64 KB of keys, 64 KB of counts)
constexpr int kHashMaxHist = kHashSlots / 2; // histories up to this long count in LDS
constexpr uint32_t kEmptySlot = 0xffffffffu;

struct PenArgs {
    int B, n_rows, V;
    float *logits;
    const int32_t *hist;
    const int32_t *hist_len;
    int hist_stride;
    const int32_t *drafts;
    int n_drafts;
    double theta, fr, pr;
    int32_t *count;   // [B][V] (long histories)
    int32_t *list;    // [B][hist_stride]: the sequence's distinct tokens
    int32_t *nlist;   // [B]: their number (long histories: in the counter region)
    int32_t *lcount;  // [B][hist_stride]: their counts (LDS-counted histories)
    int32_t *dhc;     // [B][kMaxPenDrafts]: each draft's history count (LDS-counted histories)
};

__device__ __forceinline__ uint32_t hash_slot(int t)
{
    return ((uint32_t)t * 2654435761u) >> (32 - 14);   // Fibonacci hashing onto 2^14 slots
}

__device__ __forceinline__ int hist_len_of(const PenArgs &a, int b)
{
    const int h = a.hist_len ? a.hist_len[b] : a.hist_stride;
    return min(max(h, 0), a.hist_stride);
}

// The penalized logit: these fp64 operations in this order, none fused.
__device__ __forceinline__ float penalized(float l, int c, const PenArgs &a)
{
#pragma clang fp contract(off)
    const double x = (double)l;
    const double r = x > 0.0 ? x / a.theta : x * a.theta;
    const double cf = (double)c * a.fr;
    return (float)((r - cf) - a.pr);
}

__global__ __launch_bounds__(kPenThreads) void pen_zero_kernel(PenArgs a)
{
    const int b = blockIdx.x;
    const int h = hist_len_of(a, b);
    const int64_t off = (int64_t)b * a.V;
    for (int j = blockIdx.y * kPenChunk + threadIdx.x; j < min(h, (int)(blockIdx.y + 1) * kPenChunk);
         j += kPenThreads) {
        const int t = a.hist[(int64_t)b * a.hist_stride + j];
        if (t >= 0 && t < a.V) a.count[off + t] = 0;
    }
    if (blockIdx.y == 0 && a.drafts && (int)threadIdx.x < a.n_drafts) {
        const int t = a.drafts[(int64_t)b * a.n_drafts + threadIdx.x];
        if (t >= 0 && t < a.V) a.count[off + t] = 0;
    }
}

__global__ __launch_bounds__(kPenThreads) void pen_count_kernel(PenArgs a)
{
    const int b = blockIdx.x;
    const int h = hist_len_of(a, b);
    const int64_t off = (int64_t)b * a.V;
    for (int j = blockIdx.y * kPenChunk + threadIdx.x; j < min(h, (int)(blockIdx.y + 1) * kPenChunk);
         j += kPenThreads) {
        const int t = a.hist[(int64_t)b * a.hist_stride + j];
        if (t < 0 || t >= a.V) continue;
        if (atomicAdd(&a.count[off + t], 1) == 0) a.list[(int64_t)b * a.hist_stride + atomicAdd(&a.nlist[b], 1)] = t;
    }
}

// One workgroup per sequence: its history counted in an LDS hash table (linear probing; at
// most half the slots fill, so every probe ends), written out as (token, count) pairs, and the
// history count of each drafted token.
__global__ __launch_bounds__(kHashThreads) void pen_hash_kernel(PenArgs a)
{
    __shared__ uint32_t keys[kHashSlots];
    __shared__ uint32_t cnts[kHashSlots];
    __shared__ uint32_t s_n;
    const int b = blockIdx.x, t0 = threadIdx.x;
    for (int i = t0; i < kHashSlots; i += kHashThreads) {
        keys[i] = kEmptySlot;
        cnts[i] = 0;
    }
    if (t0 == 0) s_n = 0;
    __syncthreads();
    const int h = hist_len_of(a, b);
    for (int j = t0; j < h; j += kHashThreads) {
        const int t = a.hist[(int64_t)b * a.hist_stride + j];
        if (t < 0 || t >= a.V) continue;
        uint32_t slot = hash_slot(t);
        while (true) {
            const uint32_t old = atomicCAS(&keys[slot], kEmptySlot, (uint32_t)t);
            if (old == kEmptySlot || old == (uint32_t)t) {
                atomicAdd(&cnts[slot], 1u);
                break;
            }
            slot = (slot + 1) & (kHashSlots - 1);
        }
    }
    __syncthreads();
    const int nd = a.drafts ? a.n_drafts : 0;
    if (t0 < nd) {
        const int t = a.drafts[(int64_t)b * a.n_drafts + t0];
        int c = 0;
        if (t >= 0 && t < a.V)
            for (uint32_t slot = hash_slot(t); keys[slot] != kEmptySlot; slot = (slot + 1) & (kHashSlots - 1))
                if (keys[slot] == (uint32_t)t) {
                    c = (int)cnts[slot];
                    break;
                }
        a.dhc[(int64_t)b * kMaxPenDrafts + t0] = c;
    }
    for (int i = t0; i < kHashSlots; i += kHashThreads)
        if (keys[i] != kEmptySlot) {
            const uint32_t pos = atomicAdd(&s_n, 1u);
            a.list[(int64_t)b * a.hist_stride + pos] = (int32_t)keys[i];
            a.lcount[(int64_t)b * a.hist_stride + pos] = (int32_t)cnts[i];
        }
    __syncthreads();
    if (t0 == 0) a.nlist[b] = (int32_t)s_n;
}

template <bool HASH>
__global__ __launch_bounds__(kPenThreads) void pen_apply_kernel(PenArgs a)
{
    __shared__ int sx[kMaxPenDrafts];
    const int b = blockIdx.x;
    const int nd = a.drafts ? a.n_drafts : 0;
    if ((int)threadIdx.x < nd) sx[threadIdx.x] = a.drafts[(int64_t)b * a.n_drafts + threadIdx.x];
    __syncthreads();
    float *l0 = a.logits + (int64_t)b * a.n_rows * a.V;
    const int64_t off = (int64_t)b * a.V;
    // token t with history count c0 in every row: row i adds the drafts before it
    auto apply = [&](int t, int c0) {
        int c = c0;
        for (int i = 0; i < a.n_rows; ++i) {
            if (c > 0) l0[(int64_t)i * a.V + t] = penalized(l0[(int64_t)i * a.V + t], c, a);
            if (i < nd) c += sx[i] == t;
        }
    };
    const int n = a.nlist ? a.nlist[b] : 0;
    for (int j = blockIdx.y * kPenChunk + threadIdx.x; j < min(n, (int)(blockIdx.y + 1) * kPenChunk);
         j += kPenThreads) {
        const int64_t lj = (int64_t)b * a.hist_stride + j;
        const int t = a.list[lj];
        apply(t, HASH ? a.lcount[lj] : a.count[off + t]);
    }
    if (blockIdx.y == 0 && (int)threadIdx.x < nd) {
        const int j = threadIdx.x;
        const int t = sx[j];
        bool first = t >= 0 && t < a.V;
        for (int k = 0; k < j && first; ++k) first = sx[k] != t;
        const bool in_hist = HASH ? a.dhc[(int64_t)b * kMaxPenDrafts + j] > 0 : a.count[off + t] > 0;
        if (first && !in_hist) apply(t, 0);
    }
}

__global__ void pen_clear_kernel(PenArgs a)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < a.B) a.nlist[b] = 0;
}

bool pen_shape_ok(const sv_penalty_desc *d)
{
    if (!d || d->B < 0 || d->n_rows < 0 || d->V < 1 || d->hist_stride < 0 || d->n_drafts < 0) return false;
    if (!(d->repetition > 0.0f) || d->repetition == INFINITY) return false;
    if (!(d->frequency == d->frequency) || d->frequency == INFINITY || d->frequency == -INFINITY) return false;
    if (!(d->presence == d->presence) || d->presence == INFINITY || d->presence == -INFINITY) return false;
    return true;
}

size_t pen_count_bytes(const sv_penalty_desc *d)
{
    return ((size_t)d->B * (size_t)d->V * sizeof(int32_t) + 255) & ~(size_t)255;
}

// Long histories: counts over the vocabulary, then the list.  LDS-counted ones: the list, its
// counts, its lengths and the drafts' history counts.  The workspace holds either.
size_t pen_bytes(const sv_penalty_desc *d)
{
    const size_t B = (size_t)d->B, H = (size_t)d->hist_stride;
    const size_t longh = pen_count_bytes(d) + B * H * sizeof(int32_t);
    const size_t hashed = B * (2 * H + 1 + kMaxPenDrafts) * sizeof(int32_t);
    return kCounterBytes + (longh > hashed ? longh : hashed);
}

}  // namespace

extern "C" size_t sv_penalize_workspace(const sv_penalty_desc *d)
{
    if (!pen_shape_ok(d) || d->n_drafts > kMaxPenDrafts) return 0;
    return pen_bytes(d);
}

extern "C" sv_status sv_penalize(const sv_penalty_desc *d, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!pen_shape_ok(d)) return SV_ERR_INVALID_ARG;
    if (d->n_drafts > kMaxPenDrafts) return SV_ERR_UNSUPPORTED;
    if ((int64_t)d->B * d->n_rows > 0x7fffffff || d->B > kMaxCounters) return SV_ERR_UNSUPPORTED;
    if ((int64_t)d->B * d->n_rows == 0) return SV_OK;
    if (!d->logits) return SV_ERR_INVALID_ARG;
    const bool hist = d->history && d->hist_stride > 0;
    if (!workspace || workspace_bytes < pen_bytes(d)) return SV_ERR_WORKSPACE;
    PenArgs a;
    a.B = d->B;
    a.n_rows = d->n_rows;
    a.V = d->V;
    a.logits = d->logits;
    a.hist = d->history;
    a.hist_len = d->hist_len;
    a.hist_stride = hist ? d->hist_stride : 0;
    a.drafts = d->draft_tokens;
    a.n_drafts = d->draft_tokens ? d->n_drafts : 0;
    a.theta = (double)d->repetition;
    a.fr = (double)d->frequency;
    a.pr = (double)d->presence;
    char *ws = static_cast<char *>(workspace);
    hipStream_t s = (hipStream_t)stream;
    const unsigned nchunk = hist ? (unsigned)((d->hist_stride + kPenChunk - 1) / kPenChunk) : 1u;
    if (nchunk > 65535) return SV_ERR_UNSUPPORTED;
    const dim3 g((unsigned)d->B, nchunk);
    (void)hipGetLastError();
    if (a.hist_stride <= kHashMaxHist) {
        // counted in LDS: two launches
        char *w = ws + kCounterBytes;
        const size_t BH = (size_t)d->B * (size_t)a.hist_stride * sizeof(int32_t);
        a.list = reinterpret_cast<int32_t *>(w);
        a.lcount = reinterpret_cast<int32_t *>(w + BH);
        a.nlist = reinterpret_cast<int32_t *>(w + 2 * BH);
        a.dhc = reinterpret_cast<int32_t *>(w + 2 * BH + (size_t)d->B * sizeof(int32_t));
        a.count = nullptr;
        hipLaunchKernelGGL(pen_hash_kernel, dim3((unsigned)d->B), dim3(kHashThreads), 0, s, a);
        hipLaunchKernelGGL(pen_apply_kernel<true>, g, dim3(kPenThreads), 0, s, a);
    } else {
        a.nlist = reinterpret_cast<int32_t *>(ws);
        a.count = reinterpret_cast<int32_t *>(ws + kCounterBytes);
        a.list = reinterpret_cast<int32_t *>(ws + kCounterBytes + pen_count_bytes(d));
        a.lcount = nullptr;
        a.dhc = nullptr;
        hipLaunchKernelGGL(pen_zero_kernel, g, dim3(kPenThreads), 0, s, a);
        hipLaunchKernelGGL(pen_count_kernel, g, dim3(kPenThreads), 0, s, a);
        hipLaunchKernelGGL(pen_apply_kernel<false>, g, dim3(kPenThreads), 0, s, a);
        hipLaunchKernelGGL(pen_clear_kernel, dim3((unsigned)((d->B + 255) / 256)), dim3(256), 0, s, a);
    }
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}
