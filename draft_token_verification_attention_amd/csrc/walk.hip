// walk.hip -- verification of a token tree by a walk from the root.
//
// Sources: "Speculative decoding" (Zero to Frontier textbook, ch. 20, section 20.5),
// section "Token trees check several guesses at once" (the greedy walk: move to the
// child equal to the target's choice; at the first node with no such child emit that
// choice); "Speculative-Decoding" (Medusa notes), section "Attention Tree" (under
// sampling: draw from the target at the node, look for the token among the children,
// descend level by level until no child matches).
//
// One launch per depth level, grid (chunk, sequence).  Each block reads one 2048-logit
// chunk of the row of the sequence's current node; the last block of a sequence combines
// the chunks, takes the choice (first argmax, or an inverse-CDF draw in token order with
// the Philox uniform of index = depth), looks the choice up among the node's children
// and advances the walk.  Only the rows on the walked path are read.
#include "vocab_row.h"

namespace {

using namespace sv;

// 2048 logits per block: a level reads one row, so small blocks spread it over more compute
// units (a compute unit keeps only some 32 KB of loads in flight).  Measured on the 64-node
// Medusa tree, 128,256-logit rows: 17.4 us per walk with 4096-logit blocks, 16.7 with 2048,
// 17.5 with 1024.
using WChunk = Chunk<8>;
constexpr int kChunk = WChunk::kSize;
constexpr int kMaxKids = 128;      // children of a node gathered in LDS (a node with more: full search)
constexpr int kGatherNodes = 1024;  // nodes after v that two waves scan while the choice is taken
                                    // (4680-node tree: the scan outlasted the choice, 21.5 -> 25.1 us)
constexpr int kPerThread = WChunk::kPer;

struct WalkPart {
    float m;
    int32_t arg;
    double s;
};

struct WalkWs {
    int *cnt;        // [B]
    int *cur;        // [B] node of the next level
    int *done;       // [B]
    WalkPart *part;  // [B][nchunk]
};

struct WalkArgs {
    int B, n, V, max_depth, nchunk, level;
    float kf;
    double kd;
    const float *logits;
    const int32_t *tokens, *parents;
    uint64_t seed, step;
    const uint64_t *stream_ids;
    int32_t *accept_len, *path, *out_tokens, *dev_status;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WalkLayout {
    size_t cnt, cur, done, part, total;
};

static WalkLayout walk_layout(int B, int V)
{
    const size_t nchunk = ((size_t)V + kChunk - 1) / kChunk;
    WalkLayout L;
    size_t o = 0;
    L.cnt = o;
    o += kCounterBytes;
    L.cur = o;
    o += align256((size_t)B * sizeof(int));
    L.done = o;
    o += align256((size_t)B * sizeof(int));
    L.part = o;
    o += align256((size_t)B * nchunk * sizeof(WalkPart));
    L.total = o;
    return L;
}

template <bool VEC, bool SAMPLE>
__global__ __launch_bounds__(kRowThreads) void walk_level_kernel(WalkArgs a, WalkWs w)
{
    __shared__ float fscr[kRowThreads / kWave];
    __shared__ int iscr[kRowThreads / kWave];
    __shared__ double dscr[kRowThreads / kWave];
    __shared__ double scan[kRowThreads];
    __shared__ int last_flag, s_y, s_chunk, s_nkids;
    __shared__ int s_kid[kMaxKids], s_kidtok[kMaxKids];
    __shared__ double s_base, s_target, s_factor, s_u, s_Z;
    __shared__ float s_mc, s_M;

    const int c = blockIdx.x, b = blockIdx.y;
    const int d = a.level;
    int v = 0;
    if (d > 0) {
        if (w.done[b]) return;
        v = w.cur[b];
    }
    const float *row = a.logits + ((int64_t)b * a.n + v) * a.V;
    const int base = c * kChunk;
    float x[kPerThread];
    load_chunk<VEC, kPerThread>(row, base, a.V, x);

    WalkPart part;
    if (!SAMPLE) {
        float mv = -INFINITY;
        int idx = 0x7fffffff;
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
            const int e = chunk_index<VEC>(base, k);
            if (e < a.V) argmax_merge(mv, idx, x[k], e);
        }
        block_argmax(mv, idx, fscr, iscr);
        part.m = mv;
        part.arg = idx;
        part.s = 0.0;
    } else {
        float m = -INFINITY;
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) m = fmaxf(m, x[k]);
        m = block_max(m, fscr);
        // weights in fp64 (exp2_acc; -inf logits weigh 0): the draw depends on these sums
        double s = 0.0;
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) s += exp2_acc(((double)x[k] - (double)m) * a.kd);
        s = block_sum(s, dscr);
        part.m = m;
        part.arg = 0;
        part.s = s;
    }
    if (threadIdx.x == 0) {
        WalkPart *dst = w.part + (int64_t)b * a.nchunk + c;
        st_coherent(&dst->m, part.m);
        st_coherent(&dst->arg, part.arg);
        st_coherent(&dst->s, part.s);
    }
    if (!arrive_last(&w.cnt[b], a.nchunk, &last_flag)) return;

    // ---- last block of this sequence: the choice at node v ----
    // Three things overlap: wave 0 combines the chunk partials, wave 1 (SAMPLE) draws the
    // uniform, waves 2 and 3 gather v's children and their tokens into LDS when at most
    // kGatherNodes nodes follow v (up to kMaxKids children; otherwise, and for larger trees,
    // the whole block searches the node list after the choice).
    const WalkPart *pp = w.part + (int64_t)b * a.nchunk;
    const int32_t *tk = a.tokens + (int64_t)b * a.n;
    const bool gather = a.n - (v + 1) <= kGatherNodes;
    if (threadIdx.x == 0) s_nkids = gather ? 0 : kMaxKids + 1;
    __syncthreads();
    if (gather && threadIdx.x >= 2 * kWave) {
        for (int cnode = v + 1 + (int)threadIdx.x - 2 * kWave; cnode < a.n; cnode += kRowThreads - 2 * kWave) {
            if (a.parents[cnode] == v) {
                const int slot = atomicAdd(&s_nkids, 1);
                if (slot < kMaxKids) {
                    s_kid[slot] = cnode;
                    s_kidtok[slot] = tk[cnode];
                }
            }
        }
    }
    if (!SAMPLE) {
        if (threadIdx.x < kWave) {
            float mv;
            int idx;
            wave_combine_argmax(pp, a.nchunk, mv, idx);
            if (threadIdx.x == 0) s_y = idx;
        }
        __syncthreads();
    } else {
        if (threadIdx.x < kWave) {
            float M;
            double Z;
            wave_combine_softmax(pp, a.nchunk, a.kd, M, Z);
            if (threadIdx.x == 0) {
                s_M = M;
                s_Z = Z;
            }
        } else if (threadIdx.x == kWave) {
            const uint64_t stream = a.stream_ids ? a.stream_ids[b] : (uint64_t)b;
            s_u = philox_uniform(a.seed, (uint64_t)d, a.step, stream, kTagWalk);
        }
        __syncthreads();
        if (threadIdx.x < kWave) {
            const float M = s_M;
            const double target = s_u * s_Z;
            int found;
            double cum;
            wave_find_chunk(a.nchunk, target,
                            [&](int cc) { return pp[cc].s * exp2_acc(((double)pp[cc].m - (double)M) * a.kd); }, found,
                            cum);
            if (threadIdx.x == 0) {
                s_chunk = found;
                s_base = cum;
                s_target = target;
                s_factor = exp2_acc(((double)pp[found].m - (double)M) * a.kd);
                s_mc = pp[found].m;
            }
        }
        __syncthreads();
        const int cb = s_chunk * kChunk;
        const float mc = s_mc;
        const double f = s_factor;
        auto weight = [&](float l, float) -> double { return exp2_acc(((double)l - (double)mc) * a.kd) * f; };
        int y = chunk_inverse_cdf<kPerThread, VEC>(row, nullptr, cb, a.V, s_base, s_target, weight, scan, iscr);
        if (y < 0) y = cb;  // no mass in the chunk at all (cannot happen for the chunk found)
        if (threadIdx.x == 0) s_y = y;
        __syncthreads();
    }
    const int y = s_y;

    // first child of v (in node order) whose token is y
    int child = 0x7fffffff;
    const int nkids = s_nkids;
    if (nkids <= kMaxKids) {
        if ((int)threadIdx.x < nkids && s_kidtok[threadIdx.x] == y) child = s_kid[threadIdx.x];
    } else {
        for (int cnode = v + 1 + (int)threadIdx.x; cnode < a.n; cnode += kRowThreads)
            if (a.parents[cnode] == v && tk[cnode] == y) child = min(child, cnode);
    }
    child = block_min_int(child, iscr);

    const int cap = a.max_depth + 1;
    int32_t *path = a.path + (int64_t)b * cap;
    int32_t *out = a.out_tokens + (int64_t)b * cap;
    if (d == 0) {
        for (int i = threadIdx.x; i < cap; i += kRowThreads) {
            path[i] = i == 0 ? 0 : -1;
            out[i] = -1;
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const bool has = child != 0x7fffffff;
        if (has && d + 1 <= a.max_depth) {
            path[d + 1] = child;
            out[d] = tk[child];
            w.cur[b] = child;
            w.done[b] = 0;
        } else {
            out[d] = y;
            a.accept_len[b] = d;
            w.done[b] = 1;
            if (a.dev_status) a.dev_status[b] = has ? 3 : 0;
        }
    }
}

template <bool VEC, bool SAMPLE>
static hipError_t launch_levels(const WalkArgs &a0, const WalkWs &w, hipStream_t s)
{
    WalkArgs a = a0;
    for (int d = 0; d <= a.max_depth; ++d) {
        a.level = d;
        hipLaunchKernelGGL((walk_level_kernel<VEC, SAMPLE>), dim3(a.nchunk, a.B), dim3(kRowThreads), 0, s, a, w);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

extern "C" size_t sv_tree_walk_workspace(const sv_walk_desc *d)
{
    if (!d || d->B < 0 || d->V < 1) return 0;
    return walk_layout(d->B, d->V).total;
}

extern "C" sv_status sv_tree_walk(const sv_walk_desc *d, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!d) return SV_ERR_INVALID_ARG;
    if (d->B < 0 || d->n < 1 || d->V < 1 || d->max_depth < 0) return SV_ERR_INVALID_ARG;
    if (d->mode != SV_GREEDY && d->mode != SV_SAMPLE) return SV_ERR_INVALID_ARG;
    if (!(d->temperature >= 0.0f) || d->temperature == INFINITY) return SV_ERR_INVALID_ARG;
    if (d->max_depth > 63) return SV_ERR_UNSUPPORTED;
    if (!d->logits || !d->tokens || !d->parents || !d->accept_len || !d->path || !d->out_tokens)
        return SV_ERR_INVALID_ARG;
    if (d->B == 0) return SV_OK;
    if (d->B > kMaxCounters) return SV_ERR_UNSUPPORTED;
    const WalkLayout L = walk_layout(d->B, d->V);
    if (!workspace || workspace_bytes < L.total || ((uintptr_t)workspace & 255)) return SV_ERR_WORKSPACE;
    char *ws = (char *)workspace;
    WalkWs w;
    w.cnt = (int *)(ws + L.cnt);
    w.cur = (int *)(ws + L.cur);
    w.done = (int *)(ws + L.done);
    w.part = (WalkPart *)(ws + L.part);

    const bool sample = d->mode == SV_SAMPLE && d->temperature > 0.0f;
    WalkArgs a;
    a.B = d->B;
    a.n = d->n;
    a.V = d->V;
    a.max_depth = d->max_depth;
    a.nchunk = (d->V + kChunk - 1) / kChunk;
    a.level = 0;
    a.kd = 1.4426950408889634 / (sample ? (double)d->temperature : 1.0);
    a.kf = (float)a.kd;
    a.logits = d->logits;
    a.tokens = d->tokens;
    a.parents = d->parents;
    a.seed = d->rng.seed;
    a.step = d->rng.step;
    a.stream_ids = d->rng.stream_ids;
    a.accept_len = d->accept_len;
    a.path = d->path;
    a.out_tokens = d->out_tokens;
    a.dev_status = d->dev_status;
    const bool vec = (d->V % 4 == 0) && (((uintptr_t)d->logits & 15) == 0);
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    hipError_t e;
    if (sample)
        e = vec ? launch_levels<true, true>(a, w, s) : launch_levels<false, true>(a, w, s);
    else
        e = vec ? launch_levels<true, false>(a, w, s) : launch_levels<false, false>(a, w, s);
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}
