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

// ---------------------------------------------------------------------------
// Tree verification by recursive rejection ("Speculative decoding" textbook, box
// "Recursive rejection at a node with several children"; children drawn i.i.d. from q, or
// without replacement as in the Sequoia variant the same section describes).
//
// At node v, with p, q the target's and drafter's distributions there, the residual after
// i - 1 rejections is R_i(x) = (p(x) - c_i q(x))+ / F(c_i), F(c) = sum_x (p(x) - c q(x))+,
// c_1 = 0, c_{i+1} = c_i + F(c_i) / Q_i, where Q_i is the draft mass not yet rejected (1 for
// i.i.d. children; without replacement the rejected tokens' q is removed, and their
// residual is 0 already).  Child i is tested as u q_i(s_i) < R_i(s_i), q_i = q / Q_i (0 for
// a token already rejected without replacement).  So every further try costs one pass
// over the node's two rows, to evaluate F at the next point:
//   node pass  grid (4096-token chunk, sequence): per-chunk maxima and fp64 sums of both
//              rows; the last block gets exact normalizers, the node's children in node
//              order, and tests the first child (or draws from p at a leaf).
//   try pass   grid (chunk, sequence), max_children launches per level: for sequences
//              with a rejection pending, per-chunk sums of (p - c q)+ at the next point;
//              the last block updates (c, F), tests the next child, or -- every child
//              rejected -- draws from the residual (chunk, then token in the chunk).
// State per sequence in the workspace; sequences that finished skip every later pass.
// ---------------------------------------------------------------------------
constexpr int kRrsChunk = 16 * kRowThreads;  // 4096 tokens
constexpr int kRrsPer = 16;
constexpr int kMaxRrsKids = 64;

struct RrsState {
    int node, depth, done, pending, tries, nkids;
    double Mp, Zp, Mq, Zq;   // exact maxima and normalizers of the node's rows
    double c, F, Qold, Qnew; // residual point, its mass, draft mass before and after the last rejection
    int kid[kMaxRrsKids], kidtok[kMaxRrsKids];
};
struct RrsPart {
    float mp, mq;
    double sp, sq;   // sums relative to the chunk's maxima
};

struct RrsWs {
    int *cnt;
    RrsState *st;      // [B]
    RrsPart *part;     // [B][nchunk]
    double *fpart;     // [B][nchunk]
};

struct RrsArgs {
    int B, n, V, max_depth, nchunk, level, wor, max_kids;
    double kd;
    const float *target, *draft;
    const int32_t *tokens, *parents;
    uint64_t seed, step;
    const uint64_t *stream_ids;
    int32_t *accept_len, *path, *out_tokens, *dev_status;
};

struct RrsLayout {
    size_t cnt, st, part, fpart, total;
};

static RrsLayout rrs_layout(int B, int V)
{
    const size_t nchunk = ((size_t)V + kRrsChunk - 1) / kRrsChunk;
    RrsLayout L;
    size_t o = 0;
    L.cnt = o;
    o += kCounterBytes;
    L.st = o;
    o += align256((size_t)B * sizeof(RrsState));
    L.part = o;
    o += align256((size_t)B * nchunk * sizeof(RrsPart));
    L.fpart = o;
    o += align256((size_t)B * nchunk * sizeof(double));
    L.total = o;
    return L;
}

__device__ __forceinline__ double rrs_uniform(const RrsArgs &a, int b, int d, int idx)
{
    const uint64_t stream = a.stream_ids ? a.stream_ids[b] : (uint64_t)b;
    return philox_uniform(a.seed, ((uint64_t)d << 16) | (uint64_t)idx, a.step, stream, kTagRRS);
}

// the walk moves to child `kid` (token tok) at depth d, or stops there at max_depth
__device__ void rrs_advance(const RrsArgs &a, RrsState &S, int b, int kid, int tok)
{
    const int d = S.depth;
    const int cap = a.max_depth + 1;
    a.out_tokens[(int64_t)b * cap + d] = tok;
    if (d + 1 > a.max_depth) {
        a.accept_len[b] = d;
        if (a.dev_status) a.dev_status[b] = 3;
        S.done = 1;
        return;
    }
    a.path[(int64_t)b * cap + d + 1] = kid;
    S.node = kid;
    S.depth = d + 1;
    S.pending = 0;
}

__device__ void rrs_finish(const RrsArgs &a, RrsState &S, int b, int y)
{
    a.out_tokens[(int64_t)b * (a.max_depth + 1) + S.depth] = y;
    a.accept_len[b] = S.depth;
    if (a.dev_status) a.dev_status[b] = 0;
    S.done = 1;
}

template <bool VEC>
__global__ __launch_bounds__(kRowThreads) void rrs_node_kernel(RrsArgs a, RrsWs w)
{
    __shared__ float fscr[kRowThreads / kWave];
    __shared__ double dscr[2 * (kRowThreads / kWave)];
    __shared__ double scan[kRowThreads];
    __shared__ int iscr[kRowThreads / kWave];
    __shared__ int last_flag, s_n, s_over, s_chunk;
    __shared__ int s_wcount[kRowThreads / kWave];
    __shared__ int s_kid[kMaxRrsKids], s_kidtok[kMaxRrsKids];
    __shared__ double s_Mp, s_Zp, s_Mq, s_Zq, s_u0, s_ud, s_base, s_target, s_factor;
    __shared__ float s_mc;
    const int c = blockIdx.x, b = blockIdx.y;
    RrsState &S = w.st[b];
    int v = 0;
    if (a.level > 0) {
        if (S.done) return;
        v = S.node;
    }
    const float *prow = a.target + ((int64_t)b * a.n + v) * a.V;
    const float *qrow = a.draft + ((int64_t)b * a.n + v) * a.V;
    const int base = c * kRrsChunk;
    float xp[kRrsPer], xq[kRrsPer];
    load_chunk2<VEC, kRrsPer>(prow, qrow, base, a.V, xp, xq);
    float mp = -INFINITY, mq = -INFINITY;
#pragma unroll
    for (int k = 0; k < kRrsPer; ++k) {
        mp = fmaxf(mp, xp[k]);
        mq = fmaxf(mq, xq[k]);
    }
    mp = block_max(mp, fscr);
    mq = block_max(mq, fscr);
    double sp = 0.0, sq = 0.0;
#pragma unroll
    for (int k = 0; k < kRrsPer; ++k) {
        sp += exp2_acc(((double)xp[k] - (double)mp) * a.kd);
        sq += exp2_acc(((double)xq[k] - (double)mq) * a.kd);
    }
    block_sum2(sp, sq, dscr);
    if (threadIdx.x == 0) {
        RrsPart *dst = w.part + (int64_t)b * a.nchunk + c;
        st_coherent(&dst->mp, mp);
        st_coherent(&dst->mq, mq);
        st_coherent(&dst->sp, sp);
        st_coherent(&dst->sq, sq);
    }
    if (!arrive_last(&w.cnt[b], a.nchunk, &last_flag)) return;

    // ---- last block of the sequence: exact normalizers, the children, the first try ----
    const RrsPart *pp = w.part + (int64_t)b * a.nchunk;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int d = a.level > 0 ? S.depth : 0;
    if (wave < 2) {
        float m = -INFINITY;
        for (int cc = lane; cc < a.nchunk; cc += kWave) m = fmaxf(m, wave == 0 ? pp[cc].mp : pp[cc].mq);
        m = wave_max(m);
        double z = 0.0;
        for (int cc = lane; cc < a.nchunk; cc += kWave) {
            const float mc = wave == 0 ? pp[cc].mp : pp[cc].mq;
            const double sc = wave == 0 ? pp[cc].sp : pp[cc].sq;
            if (sc > 0.0) z += sc * exp2_acc(((double)mc - (double)m) * a.kd);
        }
        z = wave_sum(z);
        if (lane == 0) {
            if (wave == 0) {
                s_Mp = m;
                s_Zp = z;
            } else {
                s_Mq = m;
                s_Zq = z;
            }
        }
    } else if (wave == 2 && lane < 2) {
        const double u = rrs_uniform(a, b, d, lane == 0 ? 0 : 0xffff);
        if (lane == 0) s_u0 = u;
        else s_ud = u;
    }
    // children of v in node order: ballot compaction over 256-node blocks
    if (threadIdx.x == 0) {
        s_n = 0;
        s_over = 0;
    }
    __syncthreads();
    const int32_t *tk = a.tokens + (int64_t)b * a.n;
    for (int c0 = v + 1; c0 < a.n; c0 += kRowThreads) {
        const int node = c0 + threadIdx.x;
        const bool is_kid = node < a.n && a.parents[node] == v;
        const uint64_t m = __ballot(is_kid);
        if (lane == 0) s_wcount[wave] = __popcll(m);
        __syncthreads();
        int before = s_n;
        for (int k = 0; k < wave; ++k) before += s_wcount[k];
        const int slot = before + __popcll(m & ((1ull << lane) - 1ull));
        if (is_kid) {
            if (slot < a.max_kids && slot < kMaxRrsKids) {
                s_kid[slot] = node;
                s_kidtok[slot] = tk[node];
            } else {
                s_over = 1;
            }
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            int tot = s_n;
            for (int k = 0; k < kRowThreads / kWave; ++k) tot += s_wcount[k];
            s_n = tot;
        }
        __syncthreads();
    }
    const int nk = min(s_n, min(a.max_kids, kMaxRrsKids));
    // the children go to the state for the try passes (later launches); this block reads LDS
    for (int k = threadIdx.x; k < nk; k += kRowThreads) {
        S.kid[k] = s_kid[k];
        S.kidtok[k] = s_kidtok[k];
    }
    if (threadIdx.x == 0) {
        if (a.level == 0) {
            S.done = 0;
            S.depth = 0;
            S.node = 0;
            const int cap = a.max_depth + 1;
            for (int i = 0; i < cap; ++i) {
                a.path[(int64_t)b * cap + i] = i == 0 ? 0 : -1;
                a.out_tokens[(int64_t)b * cap + i] = -1;
            }
        }
        S.Mp = s_Mp;
        S.Zp = s_Zp;
        S.Mq = s_Mq;
        S.Zq = s_Zq;
        S.nkids = nk;
        S.c = 0.0;
        S.F = 1.0;
        S.Qold = 1.0;
        S.Qnew = 1.0;
        S.tries = 0;
        S.pending = 0;
    }
    __syncthreads();
    if (s_over) {  // more children than max_children: status 5, the walk stops here
        if (threadIdx.x == 0) {
            a.accept_len[b] = S.depth;
            if (a.dev_status) a.dev_status[b] = 5;
            S.done = 1;
        }
        return;
    }
    if (nk > 0) {
        if (threadIdx.x == 0) {
            const int s = s_kidtok[0];
            const int sc = min(max(s, 0), a.V - 1);
            const double ps = exp2_acc(((double)prow[sc] - s_Mp) * a.kd) / s_Zp;
            const double qs = exp2_acc(((double)qrow[sc] - s_Mq) * a.kd) / s_Zq;
            if (s_u0 * qs < ps) {
                rrs_advance(a, S, b, s_kid[0], s);
            } else {
                S.tries = 1;
                S.pending = 1;
                S.Qnew = S.Qold - (a.wor ? qs : 0.0);
            }
        }
        return;
    }
    // a leaf: the extra token from p (chunk holding u Z, then the token inside it)
    if (threadIdx.x < kWave) {
        const double Mp = s_Mp;
        const double target = s_ud * s_Zp;
        int found;
        double cum;
        wave_find_chunk(a.nchunk, target,
                        [&](int cc) { return pp[cc].sp * exp2_acc(((double)pp[cc].mp - Mp) * a.kd); }, found, cum);
        if (lane == 0) {
            s_chunk = found;
            s_base = cum;
            s_target = target;
            s_factor = exp2_acc(((double)pp[found].mp - Mp) * a.kd);
            s_mc = pp[found].mp;
        }
    }
    __syncthreads();
    const float mc = s_mc;
    const double f = s_factor;
    auto weight = [&](float l, float) -> double { return exp2_acc(((double)l - (double)mc) * a.kd) * f; };
    int y = chunk_inverse_cdf<kRrsPer, VEC>(prow, nullptr, s_chunk * kRrsChunk, a.V, s_base, s_target, weight, scan,
                                            iscr);
    if (y < 0) y = s_chunk * kRrsChunk;
    if (threadIdx.x == 0) rrs_finish(a, S, b, y);
}

template <bool VEC>
__global__ __launch_bounds__(kRowThreads) void rrs_try_kernel(RrsArgs a, RrsWs w)
{
    __shared__ double dscr[kRowThreads / kWave];
    __shared__ double scan[kRowThreads];
    __shared__ int iscr[kRowThreads / kWave];
    __shared__ int last_flag, s_chunk;
    __shared__ double s_base, s_target;
    const int c = blockIdx.x, b = blockIdx.y;
    RrsState &S = w.st[b];
    if (S.done || !S.pending) return;
    const int v = S.node;
    const double Mp = S.Mp, Mq = S.Mq, iZp = 1.0 / S.Zp, iZq = 1.0 / S.Zq;
    const double cn = S.c + S.F / S.Qold;  // the next residual point
    const float *prow = a.target + ((int64_t)b * a.n + v) * a.V;
    const float *qrow = a.draft + ((int64_t)b * a.n + v) * a.V;
    float xp[kRrsPer], xq[kRrsPer];
    load_chunk2<VEC, kRrsPer>(prow, qrow, c * kRrsChunk, a.V, xp, xq);
    auto r_of = [&](float lp, float lq, double cc) {
        return fmax(0.0, exp2_acc(((double)lp - Mp) * a.kd) * iZp - cc * exp2_acc(((double)lq - Mq) * a.kd) * iZq);
    };
    double fs = 0.0;
#pragma unroll
    for (int k = 0; k < kRrsPer; ++k) fs += r_of(xp[k], xq[k], cn);
    fs = block_sum(fs, dscr);
    if (threadIdx.x == 0) st_coherent(&w.fpart[(int64_t)b * a.nchunk + c], fs);
    if (!arrive_last(&w.cnt[b], a.nchunk, &last_flag)) return;

    // ---- last block: F at the next point, then the next child or the draw ----
    const double *fp = w.fpart + (int64_t)b * a.nchunk;
    __shared__ double s_F;
    __shared__ int s_keep;
    if (threadIdx.x < kWave) {
        double f = 0.0;
        for (int cc = threadIdx.x; cc < a.nchunk; cc += kWave) f += fp[cc];
        f = wave_sum(f);
        if (threadIdx.x == 0) {
            s_keep = f > 0.0;  // F = 0 only when R = q after rounding: keep the current residual
            s_F = f;
        }
    }
    __syncthreads();
    const bool keep = s_keep != 0;
    const double cc_now = keep ? cn : S.c;
    const double F_now = keep ? s_F : S.F;
    const int i = S.tries;
    const int d = S.depth;
    if (i < S.nkids) {
        if (threadIdx.x == 0) {
            const int s = S.kidtok[i];
            const int sc = min(max(s, 0), a.V - 1);
            bool dup = false;
            if (a.wor)
                for (int j = 0; j < i; ++j) dup = dup || (S.kidtok[j] == s);
            const double ps = exp2_acc(((double)prow[sc] - Mp) * a.kd) * iZp;
            const double qs = exp2_acc(((double)qrow[sc] - Mq) * a.kd) * iZq;
            const double R = fmax(0.0, ps - cc_now * qs) / F_now;
            const double qi = a.wor ? (dup ? 0.0 : qs / S.Qnew) : qs;
            const double u = rrs_uniform(a, b, d, i);
            S.c = cc_now;
            S.F = F_now;
            if (u * qi < R) {
                rrs_advance(a, S, b, S.kid[i], s);
            } else {
                S.tries = i + 1;
                S.Qold = S.Qnew;
                S.Qnew = S.Qnew - ((a.wor && !dup) ? qs : 0.0);
            }
        }
        return;
    }
    // every child rejected: the extra token from (p - c q)+ (chunk sums of this pass)
    if (threadIdx.x < kWave) {
        const double u = rrs_uniform(a, b, d, 0xffff);
        const double target = u * F_now;
        int found;
        double cum;
        wave_find_chunk(a.nchunk, target, [&](int k) { return fp[k]; }, found, cum);
        if (threadIdx.x == 0) {
            s_chunk = found;
            s_base = cum;
            s_target = target;
        }
    }
    __syncthreads();
    auto weight = [&](float lp, float lq) -> double { return r_of(lp, lq, cc_now); };
    int y = chunk_inverse_cdf<kRrsPer, VEC>(prow, qrow, s_chunk * kRrsChunk, a.V, s_base, s_target, weight, scan,
                                            iscr);
    if (y < 0) y = s_chunk * kRrsChunk;
    if (threadIdx.x == 0) rrs_finish(a, S, b, y);
}

template <bool VEC>
static hipError_t launch_rrs(const RrsArgs &a0, const RrsWs &w, hipStream_t s)
{
    RrsArgs a = a0;
    for (int d = 0; d <= a.max_depth; ++d) {
        a.level = d;
        hipLaunchKernelGGL(rrs_node_kernel<VEC>, dim3(a.nchunk, a.B), dim3(kRowThreads), 0, s, a, w);
        for (int t = 0; t < a.max_kids; ++t)
            hipLaunchKernelGGL(rrs_try_kernel<VEC>, dim3(a.nchunk, a.B), dim3(kRowThreads), 0, s, a, w);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

extern "C" size_t sv_tree_walk_workspace(const sv_walk_desc *d)
{
    if (!d || d->B < 0 || d->V < 1) return 0;
    const bool rrs = d->mode == SV_SAMPLE && d->temperature > 0.0f && d->rule != SV_WALK_MATCH;
    return rrs ? rrs_layout(d->B, d->V).total : walk_layout(d->B, d->V).total;
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
    if (d->rule != SV_WALK_MATCH && d->rule != SV_WALK_RRS && d->rule != SV_WALK_RRS_WOR) return SV_ERR_INVALID_ARG;
    const bool rrs = d->mode == SV_SAMPLE && d->temperature > 0.0f && d->rule != SV_WALK_MATCH;
    if (rrs && (!d->draft_logits || d->max_children < 1)) return SV_ERR_INVALID_ARG;
    if (rrs && d->max_children > kMaxRrsKids) return SV_ERR_UNSUPPORTED;
    if (d->B == 0) return SV_OK;
    if (d->B > kMaxCounters) return SV_ERR_UNSUPPORTED;
    if (rrs) {
        const RrsLayout R = rrs_layout(d->B, d->V);
        if (!workspace || workspace_bytes < R.total || ((uintptr_t)workspace & 255)) return SV_ERR_WORKSPACE;
        char *ws = (char *)workspace;
        RrsWs w;
        w.cnt = (int *)(ws + R.cnt);
        w.st = (RrsState *)(ws + R.st);
        w.part = (RrsPart *)(ws + R.part);
        w.fpart = (double *)(ws + R.fpart);
        RrsArgs a;
        a.B = d->B;
        a.n = d->n;
        a.V = d->V;
        a.max_depth = d->max_depth;
        a.nchunk = (d->V + kRrsChunk - 1) / kRrsChunk;
        a.level = 0;
        a.wor = d->rule == SV_WALK_RRS_WOR;
        a.max_kids = d->max_children;
        a.kd = 1.4426950408889634 / (double)d->temperature;
        a.target = d->logits;
        a.draft = d->draft_logits;
        a.tokens = d->tokens;
        a.parents = d->parents;
        a.seed = d->rng.seed;
        a.step = d->rng.step;
        a.stream_ids = d->rng.stream_ids;
        a.accept_len = d->accept_len;
        a.path = d->path;
        a.out_tokens = d->out_tokens;
        a.dev_status = d->dev_status;
        const bool vec = (d->V % 4 == 0) && ((((uintptr_t)d->logits | (uintptr_t)d->draft_logits) & 15) == 0);
        hipStream_t s = (hipStream_t)stream;
        (void)hipGetLastError();
        const hipError_t e = vec ? launch_rrs<true>(a, w, s) : launch_rrs<false>(a, w, s);
        return e == hipSuccess ? SV_OK : SV_ERR_HIP;
    }
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
