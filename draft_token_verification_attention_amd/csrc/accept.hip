// accept.hip -- acceptance of one speculative round, vocabulary-parallel.
//
// Sources:
//   "Speculative decoding" (Zero to Frontier textbook, ch. 20, section 20.5): box "A round
//   of greedy speculative decoding"; box "The speculative sampling rule"; box "A round of
//   speculative sampling"; section "Speculative verification in PyTorch" (a zero draft row
//   after the last draft turns the bonus token into a residual draw).
//   "Speculative Decoding: The Art of Guessing Well", section "Speculative sampling".
//
// Kernels (one launch each, all decisions on the device):
//   stats    tasks (chunk, row, sequence), looping grid.  A task reads one chunk of one
//            row once and keeps, per block (4096-logit chunks) or per wave (16384-logit
//            chunks, no block-wide reduction), GREEDY (max, first argmax) or SAMPLE (max m,
//            S = sum exp((l - m)/T) in fp64).  No cross-block hand-off: the kernel
//            boundary publishes.
//   greedy   GREEDY, one block per sequence: argmax per row from the chunk partials,
//            the matching prefix J and the extra token z_J.
//   alpha    optional: sum_x min(p_i, q_i) per draft position (one more read of the rows).
//   resample SAMPLE, grid (chunk, sequence); small calls in the vector layout take
//            2048-logit chunks of their own (half the bytes per block to wait for once J
//            is known).  Every block re-derives the row statistics and the ratio tests from
//            the chunk partials in a fixed order (so all blocks agree on J), then sums the
//            residual mass of its chunk of the two rows at position J and its 256-token
//            segment sums; the last block reads every segment sum at once and finds the
//            segment holding u* Z (block-wide scan), then (one wave, token order) the extra
//            token.  When the residual has no mass, or the layout is not the vector one, it
//            finds the chunk first, then the token inside it.
// Exponentials of the statistics pass (and of the optional alpha pass) run in fp32: their
// normalizers are good to about 1e-9, ample for the ratio tests.  The decided p(x), q(x),
// the residual and CDF weights, and the normalizers the draw uses are fp64 (exp, exp2_acc),
// and so is every sum.
#include <mutex>

#include "vocab_row.h"

namespace {

using namespace sv;

// A block reads 4096 (PER = 16) or 16384 (PER = 64) logits of one row, all loaded
// before any reduction: the larger chunk when the call has blocks to spare (big batches),
// the smaller one when latency matters (a single sequence).
constexpr int kMinChunk = 16 * kRowThreads;
// Row partials per chunk: with the large chunks (big calls) every wave keeps its own (no
// block barrier per task, for bandwidth); with the small ones (latency) the block reduces to
// one, which keeps the decide step's staging small.
template <int PER>
constexpr int parts_per_chunk() { return PER >= 64 ? kRowThreads / kWave : 1; }
constexpr int kMaxPartsPerChunk = kRowThreads / kWave;
// The residual draw of a small call (vector layout) takes 2048-logit chunks: twice the
// blocks of the stats chunks, half the bytes each block waits for once J is known.
constexpr int kResPer = 8;
constexpr int kResChunk = kResPer * kRowThreads;

struct RowPart {
    float m;
    int32_t arg;
    double s;
};
struct ResPart {   // per residual chunk: sums of wp and wq over the tokens with residual
    double a, b;    // mass (estimated), and of wp and wq over every token of the chunk
    double wp, wq;
};

struct BlockChunk {   // block verification, per (sequence, candidate, 4096-token chunk)
    double a, b;      // sums of wp and wq over the tokens with (estimated) residual mass
    double wp, wq;    // sums of wp and wq over every token
};
struct GumbelPart {   // Gumbel-coupled verification, per (sequence, position, chunk)
    double s;         // the chunk's best score l/T + g
    int32_t arg;      // its token (the lowest among equal scores)
    int32_t pad;
};
constexpr int kBlockPer = 16;  // block verification and Gumbel passes: 4096-token chunks
constexpr int kBlockChunk = kBlockPer * kRowThreads;

struct AcceptWs {
    int *cnt;        // [B]: one completion counter per sequence, shared by the call's kernels in turn
    RowPart *part;   // [B][rows][npart]: one partial per (chunk, wave)
    double *u;       // [B][gamma + 1]: the round's uniforms (ratio tests, then the extra token)
    ResPart *res;    // [B][nchunk]
    double *seg;     // [B][nchunk][PER][2]: (A, B) of each 256-token segment of a chunk
    double *apart;   // [B][gamma][nchunk]
    BlockChunk *bchunk;  // block verification: [B][gamma + 1][4096-token chunks]
    double *bseg;        // block verification: [B][gamma + 1][chunks][16][2] (A, B per segment)
    GumbelPart *gpart;   // Gumbel coupling: [B][gamma + 1][4096-token chunks]
};

struct AcceptArgs {
    int B, gamma, V, rows, nchunk;
    int rnchunk;       // chunks of the residual draw (its own chunk size)
    int npart;         // row partials: nchunk x waves per block
    int sample;
    float kf;          // log2(e) / T in fp32, for the bulk exponentials
    double inv_t;      // 1 / T in fp64, for decided probabilities
    double kd;         // log2(e) / T in fp64, for chunk rescaling
    double tau;        // T in fp64 (Gumbel scores l / T)
    int rule;          // sv_rule
    const float *target, *draft;
    const int32_t *tokens;
    uint64_t seed, step;
    const uint64_t *stream_ids;
    int32_t *accept_len, *out_tokens, *dev_status;
    float *alpha;
    const int32_t *draft_len;  // or NULL: every sequence verifies gamma drafts
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
    size_t cnt, part, u, res, seg, apart, bchunk, bseg, gchunk, total;
};

static WsLayout accept_layout(int B, int gamma, int V, int rule = SV_RULE_TOKEN)
{
    const size_t rows = 2 * (size_t)gamma + 1;
    const size_t nchunk = ((size_t)V + kMinChunk - 1) / kMinChunk;  // the larger of the two chunk counts
    WsLayout L;
    size_t o = 0;
    L.cnt = o;
    o += kCounterBytes;
    L.part = o;
    o += align256((size_t)B * rows * nchunk * kMaxPartsPerChunk * sizeof(RowPart));
    L.u = o;
    o += align256((size_t)B * (gamma + 1) * sizeof(double));
    L.res = o;  // per resample chunk: the smallest chunks are kResChunk tokens
    o += align256((size_t)B * (((size_t)V + kResChunk - 1) / kResChunk) * sizeof(ResPart));
    L.seg = o;  // (A, B) of every 256-token segment: enough for either chunk size
    o += align256((size_t)B * (nchunk + 3) * 16 * 2 * sizeof(double));
    L.apart = o;
    o += align256((size_t)B * gamma * nchunk * sizeof(double));
    const size_t bnchunk = ((size_t)V + kBlockChunk - 1) / kBlockChunk;
    L.bchunk = o;
    if (rule == SV_RULE_BLOCK) o += align256((size_t)B * (gamma + 1) * bnchunk * sizeof(BlockChunk));
    L.bseg = o;
    if (rule == SV_RULE_BLOCK) o += align256((size_t)B * (gamma + 1) * bnchunk * kBlockPer * 2 * sizeof(double));
    L.gchunk = o;
    if (rule == SV_RULE_GUMBEL) o += align256((size_t)B * (gamma + 1) * bnchunk * sizeof(GumbelPart));
    L.total = o;
    return L;
}

// Segment sums a thread of the resample's last block reads at once (sequences of up to
// 256 x 4 segments of 256 tokens take the one-pass segment search)
constexpr int kSegPerThread = 4;

// Row partials staged in LDS by the decide steps (dynamic shared memory, at most this many)
constexpr int kMaxStaged = 2048;

__device__ __forceinline__ const float *row_ptr(const AcceptArgs &a, int b, int r)
{
    if (r <= a.gamma) return a.target + ((int64_t)b * (a.gamma + 1) + r) * a.V;
    return a.draft + ((int64_t)b * a.gamma + (r - a.gamma - 1)) * a.V;
}

__device__ __forceinline__ uint64_t stream_of(const AcceptArgs &a, int b)
{
    return a.stream_ids ? a.stream_ids[b] : (uint64_t)b;
}

// The drafts sequence b verifies (its own gamma): draft_len[b], taken into [0, gamma] (a
// length outside it is reported by the decide step), or gamma without per-sequence lengths.
// Sequence b then gets exactly the round the rule gives with gamma = its length, on its
// first rows; rows past them are neither read nor needed.
__device__ __forceinline__ int gamma_of(const AcceptArgs &a, int b)
{
    return a.draft_len ? min(max(a.draft_len[b], 0), a.gamma) : a.gamma;
}
// dev_status of sequence b: 3 for a length outside [0, gamma], else 2 for a verified draft
// token outside [0, V), else 0
__device__ __forceinline__ int32_t status_of(const AcceptArgs &a, int b, bool bad_token)
{
    if (a.draft_len && (a.draft_len[b] < 0 || a.draft_len[b] > a.gamma)) return 3;
    return bad_token ? 2 : 0;
}

// ---------------------------------------------------------------------------
// Row statistics from the chunk partials, identical in every block that computes them:
// the partials of rows [0, nrows) are staged in LDS (one memory round trip), then one
// wave per row reduces them in a fixed lane order.
// ---------------------------------------------------------------------------
// Stage the n chunk partials of a sequence in LDS (n <= kMaxStaged).  Every thread
// issues NT unconditional loads (clamped in-bounds addresses) before any is waited for;
// `meanwhile` runs between issuing them and using them.
template <int NT, typename Fn>
__device__ __forceinline__ void stage_parts_nt(const RowPart *pp, int n, RowPart *stage, Fn meanwhile)
{
    // moved as raw 16-byte vectors (an array of the struct would live in private memory)
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    static_assert(sizeof(RowPart) == sizeof(u32x4), "16-byte partials");
    const u32x4 *src = reinterpret_cast<const u32x4 *>(pp);
    u32x4 *dst = reinterpret_cast<u32x4 *>(stage);
    u32x4 t[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) t[u] = src[min((int)threadIdx.x + u * kRowThreads, n - 1)];
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of `meanwhile`
    meanwhile();
    // unconditional stores (the stage has NT * kRowThreads slots): a conditional store
    // would let the compiler sink its load next to it, one round trip per load
#pragma unroll
    for (int u = 0; u < NT; ++u) dst[threadIdx.x + u * kRowThreads] = t[u];
    __syncthreads();
}

template <typename Fn>
__device__ __forceinline__ void stage_parts(const RowPart *pp, int n, RowPart *stage, Fn meanwhile)
{
    static_assert(kMaxStaged <= 8 * kRowThreads, "staging depth");
    if (n <= kRowThreads)
        stage_parts_nt<1>(pp, n, stage, meanwhile);
    else if (n <= 2 * kRowThreads)
        stage_parts_nt<2>(pp, n, stage, meanwhile);
    else if (n <= 4 * kRowThreads)
        stage_parts_nt<4>(pp, n, stage, meanwhile);
    else
        stage_parts_nt<8>(pp, n, stage, meanwhile);
}

template <int LPR>
__device__ __forceinline__ void row_softmax_stats_lpr(const RowPart *src, int nrows, int nchunk, double kd,
                                                      double *sM, double *sZ)
{
    constexpr int RPP = kRowThreads / LPR;  // rows per block pass
    const int lane_row = (int)threadIdx.x / LPR;
    for (int r0 = 0; r0 < nrows; r0 += RPP) {
        float M;
        double Z;
        group_combine_softmax<LPR>(src, r0 + lane_row, nrows, nchunk, kd, M, Z);
        if ((threadIdx.x % LPR) == 0 && r0 + lane_row < nrows) {
            sM[r0 + lane_row] = (double)M;
            sZ[r0 + lane_row] = Z;
        }
    }
    __syncthreads();
}

// (M, Z) of rows [0, nrows): the chunk partials of a row sit on 16, 32 or 64 lanes -- the
// fewest lanes that hold a part each, but more lanes per row only while every row still
// fits in one pass of the block (a second pass costs more than a lane reading two parts)
__device__ __forceinline__ void row_softmax_stats(const RowPart *src, int nrows, int nchunk, double kd, double *sM,
                                                  double *sZ)
{
    if (nchunk <= 16 || nrows > kRowThreads / 32)
        row_softmax_stats_lpr<16>(src, nrows, nchunk, kd, sM, sZ);
    else if (nchunk <= 32 || nrows > kRowThreads / 64)
        row_softmax_stats_lpr<32>(src, nrows, nchunk, kd, sM, sZ);
    else
        row_softmax_stats_lpr<64>(src, nrows, nchunk, kd, sM, sZ);
}

// ---------------------------------------------------------------------------
template <bool VEC, bool SAMPLE, int PER>
__global__ __launch_bounds__(kRowThreads) void accept_stats_kernel(AcceptArgs a, AcceptWs w)
{
    constexpr int kChunk = PER * kRowThreads;
    constexpr int kPerThread = PER;
    __shared__ float fscr[kRowThreads / kWave];
    __shared__ int iscr[kRowThreads / kWave];
    __shared__ double dscr[kRowThreads / kWave];
    const int g = a.gamma;
    // Tasks (chunk, row, sequence), chunk fastest; SAMPLE adds one row of tasks per
    // sequence that draws the round's uniforms.  A grid smaller than the task count loops
    // over them (blocks stay resident instead of being dispatched one per task).
    const int rows_t = a.rows + (SAMPLE ? 1 : 0);
    const int ntask = a.nchunk * rows_t * a.B;
    // Block 0 also zeroes the call's completion counters, which only the later kernels of
    // the call use: a workspace is then ready whatever an earlier call left in it.
    if (blockIdx.x == 0)
        for (int b = threadIdx.x; b < a.B; b += kRowThreads) w.cnt[b] = 0;
    for (int t = blockIdx.x; t < ntask; t += gridDim.x) {
        const int c = t % a.nchunk;
        const int r = (t / a.nchunk) % rows_t;
        const int b = t / (a.nchunk * rows_t);
        if (SAMPLE && r == a.rows) {
            // the uniforms depend on no data: drawn off the decide step's critical path
            if (c == 0 && (int)threadIdx.x <= g)
                w.u[(int64_t)b * (g + 1) + threadIdx.x] =
                    philox_uniform(a.seed, threadIdx.x, a.step, stream_of(a, b), kTagAccept);
            continue;
        }
        // rows past the sequence's own length are not needed (target row gb is its last)
        if (a.draft_len) {
            const int gb = gamma_of(a, b);
            if (r <= g ? r > gb : r - g - 1 >= gb) continue;
        }
        const float *row = row_ptr(a, b, r);
        const int base = c * kChunk;
        float xv[kPerThread];
        load_chunk<VEC, kPerThread>(row, base, a.V, xv);

        constexpr int kParts = parts_per_chunk<PER>();
        RowPart part;
        if (!SAMPLE) {
            float v = -INFINITY;
            int idx = 0x7fffffff;
#pragma unroll
            for (int k = 0; k < kPerThread; ++k) argmax_merge(v, idx, xv[k], chunk_index<VEC>(base, k));
            // positions beyond V hold -inf and never win
            if (kParts > 1)
                wave_argmax(v, idx);
            else
                block_argmax(v, idx, fscr, iscr);
            part.m = v;
            part.arg = idx;
            part.s = 0.0;
        } else {
            // each thread: its own max and its sum relative to it (no barrier); then the
            // block rescales the per-thread sums to the chunk max.  fp32 exponentials: these
            // normalizers (good to about 1e-9) serve the ratio tests, whose tolerance is
            // 1e-6, and tell the residual draw which tokens carry residual mass; the draw
            // itself weighs that mass with exact normalizers of its own.
            float mt = -INFINITY;
#pragma unroll
            for (int k = 0; k < kPerThread; ++k) mt = fmaxf(mt, xv[k]);
            // branch-free: -inf logits (masked, or beyond V) weigh exp2_fast(-inf) = 0
            const float mref = mt == -INFINITY ? 0.0f : mt;
            double st = 0.0;
#pragma unroll
            for (int k = 0; k < kPerThread; ++k) st += (double)exp2_fast((xv[k] - mref) * a.kf);
            const float m = kParts > 1 ? wave_max(mt) : block_max(mt, fscr);
            const double z = st > 0.0 ? st * (double)exp2_fast((mt - m) * a.kf) : 0.0;
            const double sm = kParts > 1 ? wave_sum(z) : block_sum(z, dscr);
            part.m = m;
            part.arg = 0;
            part.s = sm;
        }
        if ((kParts > 1 && threadIdx.x % kWave == 0) || threadIdx.x == 0)
            w.part[((int64_t)b * a.rows + r) * a.npart + c * kParts + threadIdx.x / kWave] = part;
    }
}

// ---------------------------------------------------------------------------
// GREEDY decide, one block per sequence: z_i = argmax of target row i, J = the length of
// the prefix with x_i == z_i, emitted x_0..x_{J-1}, z_J.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kRowThreads) void accept_greedy_kernel(AcceptArgs a, AcceptWs w)
{
    extern __shared__ __align__(16) unsigned char dyn_lds[];
    __shared__ int z[65];
    __shared__ int firstbad, bad;
    const int b = blockIdx.x;
    const int g = a.gamma;
    const int gb = gamma_of(a, b);
    const int x = threadIdx.x < g ? a.tokens[(int64_t)b * g + threadIdx.x] : 0;
    if (threadIdx.x == 0) {
        firstbad = gb;
        bad = 0;
    }
    const RowPart *pp = w.part + (int64_t)b * a.rows * a.npart;
    RowPart *stage = reinterpret_cast<RowPart *>(dyn_lds);
    const bool staged = a.rows * a.npart <= kMaxStaged;
    if (staged) stage_parts(pp, a.rows * a.npart, stage, [] {});
    const int wave = threadIdx.x / kWave;
    for (int r = wave; r <= gb; r += kRowThreads / kWave) {
        float v;
        int idx;
        if (staged)
            wave_combine_argmax(stage + (int64_t)r * a.npart, a.npart, v, idx);
        else
            wave_combine_argmax(pp + (int64_t)r * a.npart, a.npart, v, idx);
        if (threadIdx.x % kWave == 0) z[r] = idx;
    }
    __syncthreads();
    if ((int)threadIdx.x < gb) {
        if (x != z[threadIdx.x]) atomicMin(&firstbad, (int)threadIdx.x);
        if (x < 0 || x >= a.V) bad = 1;
    }
    __syncthreads();
    const int J = firstbad;
    int32_t *out = a.out_tokens + (int64_t)b * (g + 1);
    for (int i = threadIdx.x; i <= g; i += blockDim.x) out[i] = i < J ? a.tokens[(int64_t)b * g + i] : (i == J ? z[J] : -1);
    if (a.alpha)  // alpha is a sampling quantity
        for (int i = threadIdx.x; i < g; i += blockDim.x) a.alpha[(int64_t)b * g + i] = __int_as_float(0x7fc00000);
    if (threadIdx.x == 0) {
        a.accept_len[b] = J;
        if (a.dev_status) a.dev_status[b] = status_of(a, b, bad);
    }
}

// ---------------------------------------------------------------------------
template <bool VEC, int PER>
__global__ __launch_bounds__(kRowThreads) void accept_alpha_kernel(AcceptArgs a, AcceptWs w)
{
    constexpr int kChunk = PER * kRowThreads;
    constexpr int kPerThread = PER;
    __shared__ double dscr[kRowThreads / kWave];
    __shared__ double sM[2], sZ[2];
    __shared__ int last_flag;
    const int c = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
    const int g = a.gamma;
    const int gb = gamma_of(a, b);
    // a position past the sequence's length is not verified: it adds nothing and its alpha
    // is NaN (its block still arrives at the counter)
    const bool live = i < gb;
    float xp[kPerThread], xq[kPerThread];
    const int base = c * kChunk;
    const int ir = live ? i : 0;
    load_chunk2<VEC, kPerThread>(row_ptr(a, b, ir), row_ptr(a, b, g + 1 + ir), base, a.V, xp, xq);
    // statistics of rows i (target) and gamma+1+i (draft): waves 0 and 1
    const int wave = threadIdx.x / kWave;
    if (wave < 2) {
        float M;
        double Z;
        group_combine_softmax<kWave>(w.part + ((int64_t)b * a.rows + (wave == 0 ? ir : g + 1 + ir)) * a.npart, 0, 1,
                                     a.npart, a.kd, M, Z);
        if (threadIdx.x % kWave == 0) {
            sM[wave] = (double)M;
            sZ[wave] = Z;
        }
    }
    __syncthreads();
    const float Mp = (float)sM[0], Mq = (float)sM[1];
    const double iZp = 1.0 / sZ[0], iZq = 1.0 / sZ[1];
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        if (xp[k] == -INFINITY && xq[k] == -INFINITY) continue;
        const double p = (double)exp2_fast((xp[k] - Mp) * a.kf) * iZp;
        const double q = (double)exp2_fast((xq[k] - Mq) * a.kf) * iZq;
        s += fmin(p, q);
    }
    s = block_sum(s, dscr);
    if (threadIdx.x == 0) st_coherent(&w.apart[((int64_t)b * g + i) * a.nchunk + c], live ? s : 0.0);
    if (!arrive_last(&w.cnt[b], g * a.nchunk, &last_flag)) return;
    for (int j = threadIdx.x; j < g; j += blockDim.x) {
        double t = 0.0;
        for (int cc = 0; cc < a.nchunk; ++cc) t += w.apart[((int64_t)b * g + j) * a.nchunk + cc];
        a.alpha[(int64_t)b * g + j] = j < gb ? (float)t : __int_as_float(0x7fc00000);
    }
}

// ---------------------------------------------------------------------------
// SAMPLE decide and residual draw.  Every block of sequence b: row statistics of the
// 2 gamma + 1 rows, the ratio tests u_i q(x_i) < p(x_i) (all blocks reach the same J),
// then the residual mass of its chunks of the rows at position J (chunks x, x + X, ... for
// block x of X: a grid that fits on the GPU at once, each block taking the statistics and
// the ratio tests once for several chunks).
// ---------------------------------------------------------------------------
// (two waves per SIMD: left unbounded, the large-chunk form takes more than 256 registers and
// runs one wave per SIMD, 28 -> 35 us on the 64-sequence batch)
template <bool VEC, int PER>
__global__ __launch_bounds__(kRowThreads, 2) void accept_resample_kernel(AcceptArgs a, AcceptWs w)
{
    constexpr int kChunk = PER * kRowThreads;
    constexpr int kPerThread = PER;
    extern __shared__ __align__(16) unsigned char dyn_lds[];
    __shared__ double sM[129], sZ[129];
    __shared__ double dscr[2 * (kRowThreads / kWave)];
    __shared__ double scan[kRowThreads];
    __shared__ int iscr[kRowThreads / kWave];
    __shared__ int last_flag, s_chunk, s_usep, s_seg0, firstbad, bad;
    __shared__ int s_whit[kRowThreads / kWave], s_wlast[kRowThreads / kWave];
    __shared__ double s_base, s_target, s_uextra;
    const int b = blockIdx.y;
    const int g = a.gamma;
    const int gb = gamma_of(a, b);  // this sequence's drafts (rows past them are not read)

    // drafted tokens and their logits (two dependent loads, hidden behind the staging of the
    // row partials and the row statistics; a bad token is flagged below, its logit unused),
    // and the uniforms: thread i < gamma ratio test i, thread gamma the extra token.
    // Unconditional loads from clamped slots: a load under a branch would be waited for at
    // the branch, before the partials are asked for.
    const int ti = min((int)threadIdx.x, g - 1);
    const int x = a.tokens[(int64_t)b * g + ti];
    const int xc = min(max(x, 0), a.V - 1);
    const float lpx = a.target[((int64_t)b * (g + 1) + ti) * a.V + xc];
    const float lqx = a.draft[((int64_t)b * g + ti) * a.V + xc];
    const double u_mine = w.u[(int64_t)b * (g + 1) + min((int)threadIdx.x, g)];
    if (threadIdx.x == 0) {
        firstbad = gb;
        bad = 0;
    }
    const RowPart *pp = w.part + (int64_t)b * a.rows * a.npart;
    RowPart *stage = reinterpret_cast<RowPart *>(dyn_lds);
    auto keep_extra = [&] {
        if ((int)threadIdx.x == gb) s_uextra = u_mine;
    };
    if (a.rows * a.npart <= kMaxStaged) {
        stage_parts(pp, a.rows * a.npart, stage, keep_extra);
        row_softmax_stats(stage, a.rows, a.npart, a.kd, sM, sZ);
    } else {
        keep_extra();
        __syncthreads();
        row_softmax_stats(pp, a.rows, a.npart, a.kd, sM, sZ);
    }
    if ((int)threadIdx.x < gb) {
        const int i = threadIdx.x;
        bool pass = false;
        if (x >= 0 && x < a.V) {
            const double p = exp(((double)lpx - sM[i]) * a.inv_t) / sZ[i];
            const double q = exp(((double)lqx - sM[g + 1 + i]) * a.inv_t) / sZ[g + 1 + i];
            pass = u_mine * q < p;
        } else {
            bad = 1;
        }
        if (!pass) atomicMin(&firstbad, i);
    }
    __syncthreads();
    const int J = firstbad;
    if (blockIdx.x == 0) {
        int32_t *out = a.out_tokens + (int64_t)b * (g + 1);
        for (int i = threadIdx.x; i <= g; i += blockDim.x)
            if (i != J) out[i] = i < J ? a.tokens[(int64_t)b * g + i] : -1;
        if (threadIdx.x == 0) {
            a.accept_len[b] = J;
            if (a.dev_status) a.dev_status[b] = status_of(a, b, bad);
        }
    }

    const float *prow = a.target + ((int64_t)b * (g + 1) + J) * a.V;
    const float *qrow = J < gb ? a.draft + ((int64_t)b * g + J) * a.V : nullptr;

    // Weights of token e relative to the rows' maxima, in fp64 (exp2_acc):
    // wp = 2^((l_p(e) - Mp) k), wq likewise (0 with no draft row, J == gamma).  The residual is
    // r(e) = max(0, wp/Zp - wq/Zq) with the normalizers Zp = sum wp, Zq = sum wq, which only
    // the last block knows exactly (every block sums its chunk of both rows).  The statistics
    // pass gives them to about 1e-9 (fp32 exponentials): enough to tell which tokens carry
    // residual mass (wp/Zp' > wq/Zq'), not to weigh it.  So every block stores, per 256-token
    // segment and per chunk, the sums A = sum wp and B = sum wq over those tokens, and the
    // chunk's totals of wp and wq; the last block weighs a segment as A/Zp - B/Zq with the
    // exact normalizers.  (A token misjudged by the estimate holds a residual smaller than the
    // estimate's error: the segment masses are off by its square.)
    const double Mp = sM[J], Mq = J < gb ? sM[g + 1 + J] : Mp;
    const double iZp_est = 1.0 / sZ[J], iZq_est = J < gb ? 1.0 / sZ[g + 1 + J] : 0.0;
    const double qmask = J < gb ? 1.0 : 0.0;
    // (l - M) kd as one multiply-add on the precomputed -M kd: 1e-16 |M kd| more error in
    // the exponent, ~1e-14 of a weight at logits of 100, one instruction less per weight
    const double nMpk = -Mp * a.kd, nMqk = -Mq * a.kd;
    auto wp_of = [&](float l) { return exp2_acc(fma((double)l, a.kd, nMpk)); };
    auto wq_of = [&](float l) { return exp2_acc(fma((double)l, a.kd, nMqk)) * qmask; };

    for (int c = blockIdx.x; c < a.rnchunk; c += gridDim.x) {
        const int base = c * kChunk;
        float xp[kPerThread], xq[kPerThread];
        load_chunk2<VEC, kPerThread>(prow, qrow ? qrow : prow, base, a.V, xp, xq);
        // branch-free: a position at or beyond V holds -inf, whose weight is 0.  Per thread, the
        // sums of each float4 group (VEC layout: group k4 of wave w is part of the chunk's
        // 256-token segment 4 k4 + w, in token order)
        double ta = 0.0, tb = 0.0, tp = 0.0, tq = 0.0;
        double a4[kPerThread / 4], b4[kPerThread / 4];
#pragma unroll
        for (int k4 = 0; k4 < kPerThread / 4; ++k4) {
            a4[k4] = 0.0;
            b4[k4] = 0.0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const double wp = wp_of(xp[4 * k4 + j]), wq = wq_of(xq[4 * k4 + j]);
                tp += wp;
                tq += wq;
                const bool in = wp * iZp_est > wq * iZq_est;
                a4[k4] += in ? wp : 0.0;
                b4[k4] += in ? wq : 0.0;
            }
            ta += a4[k4];
            tb += b4[k4];
        }
        if (VEC) {
            const int wv = threadIdx.x / kWave;
            double *sg = w.seg + 2 * (((int64_t)b * a.rnchunk + c) * kPerThread);
#pragma unroll
            for (int k4 = 0; k4 < kPerThread / 4; ++k4) {
                const double sa = wave_sum(a4[k4]), sb = wave_sum(b4[k4]);
                if (threadIdx.x % kWave == 0) {
                    st_coherent(&sg[2 * (4 * k4 + wv)], sa);
                    st_coherent(&sg[2 * (4 * k4 + wv) + 1], sb);
                }
            }
        }
        block_sum2(ta, tb, dscr);
        block_sum2(tp, tq, dscr);
        if (threadIdx.x == 0) {
            ResPart *rp = &w.res[(int64_t)b * a.rnchunk + c];
            st_coherent(&rp->a, ta);
            st_coherent(&rp->b, tb);
            st_coherent(&rp->wp, tp);
            st_coherent(&rp->wq, tq);
        }
    }
    if (!arrive_last(&w.cnt[b], gridDim.x, &last_flag)) return;

    // ---- last block: the exact normalizers, then the extra token ----
    const ResPart *rp = w.res + (int64_t)b * a.rnchunk;
    // (every thread's share of the chunk totals, loaded first: their sum gates all the rest)
    double zp = 0.0, zq = 0.0;
    for (int cc = threadIdx.x; cc < a.rnchunk; cc += kRowThreads) {
        zp += rp[cc].wp;
        zq += rp[cc].wq;
    }
    // wave 0, the residual's 256-token segment starting at token seg0 holding u* Z, whose
    // mass before it is sbase: the token inside it (every lane returns it)
    double iZp = 0.0, iZq = 0.0;
    auto r_of = [&](float lp, float lq) { return fmax(0.0, wp_of(lp) * iZp - wq_of(lq) * iZq); };
    auto token_in_segment = [&](int seg0, double sbase, double target) -> int {
        const int lane = threadIdx.x;
        const int e0 = seg0 + 4 * lane;  // this lane's four tokens
        const int ec = min(e0, a.V - 4);
        const float4 fp = *reinterpret_cast<const float4 *>(prow + ec);
        const float4 fq = *reinterpret_cast<const float4 *>((qrow ? qrow : prow) + ec);
        const bool in = e0 < a.V;
        double wt[4];
        wt[0] = in ? r_of(fp.x, fq.x) : 0.0;
        wt[1] = in ? r_of(fp.y, fq.y) : 0.0;
        wt[2] = in ? r_of(fp.z, fq.z) : 0.0;
        wt[3] = in ? r_of(fp.w, fq.w) : 0.0;
        const double lsum = ((wt[0] + wt[1]) + wt[2]) + wt[3];
        const double c0 = sbase + wave_scan_incl(lsum, 0.0, OpAdd()) - lsum;
        int hit = -1, lastpos = -1;
        double pre = c0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pre += wt[j];
            if (hit < 0 && pre > target && wt[j] > 0.0) hit = j;
            if (wt[j] > 0.0) lastpos = j;
        }
        const uint64_t hm = __ballot(c0 <= target && hit >= 0);
        const uint64_t lm = __ballot(lastpos >= 0);
        int y;
        if (hm) {
            const int hl = __ffsll((unsigned long long)hm) - 1;
            y = seg0 + 4 * hl + lane_value(hit, hl);
        } else if (lm) {  // rounding: the segment's running sum stops short of target
            const int ll = 63 - __clzll((unsigned long long)lm);
            y = seg0 + 4 * ll + lane_value(lastpos, ll);
        } else {
            y = seg0;  // no mass in the segment at all (cannot happen for the segment found)
        }
        return y;
    };

    // last block, residual with mass (the common case): the block reads every 256-token
    // segment's (A, B) of the sequence at once (kSegPerThread consecutive segments per
    // thread, so in token order, coalesced), weighs them with the exact normalizers, scans
    // them, finds the segment holding u* Z_r with Z_r their total, and wave 0 finds the token
    // inside it
    if (VEC && a.rnchunk * kPerThread <= kRowThreads * kSegPerThread) {
        static_assert(kSegPerThread == 4 && kPerThread % kSegPerThread == 0, "whole threads of segments");
        const int t = threadIdx.x, lane = t % kWave, wv = t / kWave;
        const int nseg = a.rnchunk * kPerThread;
        const bool live = t * kSegPerThread < nseg;
        // four unconditional 16-byte loads (A, B of four segments) from a clamped thread
        const double2 *sg = reinterpret_cast<const double2 *>(
            w.seg + 2 * ((int64_t)b * nseg + (int64_t)min(t, nseg / kSegPerThread - 1) * kSegPerThread));
        const double2 h0 = sg[0], h1 = sg[1], h2 = sg[2], h3 = sg[3];
        block_sum2(zp, zq, dscr);
        iZp = 1.0 / zp;
        iZq = qrow ? 1.0 / zq : 0.0;
        const double2 hs[kSegPerThread] = {h0, h1, h2, h3};
        double v[kSegPerThread];
#pragma unroll
        for (int j = 0; j < kSegPerThread; ++j) v[j] = live ? fmax(0.0, hs[j].x * iZp - hs[j].y * iZq) : 0.0;
        const double ts = ((v[0] + v[1]) + v[2]) + v[3];
        const double incl_w = wave_scan_incl(ts, 0.0, OpAdd());
        __syncthreads();  // dscr is reused below
        if (lane == kWave - 1) dscr[wv] = incl_w;
        __syncthreads();
        double wbase = 0.0, zr = 0.0;
#pragma unroll
        for (int k = 0; k < kRowThreads / kWave; ++k) {
            if (k < wv) wbase += dscr[k];
            zr += dscr[k];
        }
        if (zr > 0.0) {  // the same in every thread
            const double incl = wbase + incl_w;
            const double target = s_uextra * zr;
            const uint64_t hit = __ballot(ts > 0.0 && incl > target);
            const uint64_t pos = __ballot(ts > 0.0);
            if (lane == 0) {
                s_whit[wv] = hit ? wv * kWave + __ffsll((unsigned long long)hit) - 1 : kRowThreads;
                s_wlast[wv] = pos ? wv * kWave + 63 - __clzll((unsigned long long)pos) : -1;
            }
            __syncthreads();
            int th = kRowThreads, tl = -1;
#pragma unroll
            for (int k = 0; k < kRowThreads / kWave; ++k) {
                th = min(th, s_whit[k]);
                tl = max(tl, s_wlast[k]);
            }
            // rounding can leave every running sum at or below target: the last thread with mass
            if (t == (th < kRowThreads ? th : tl)) {
                double cum = incl - ts;
                int sj = -1, lastj = 0;
                double sbase = cum, lastbase = cum;
#pragma unroll
                for (int j = 0; j < kSegPerThread; ++j) {
                    if (v[j] > 0.0) {
                        if (sj < 0 && cum + v[j] > target) {
                            sj = j;
                            sbase = cum;
                        }
                        lastj = j;
                        lastbase = cum;
                    }
                    cum += v[j];
                }
                if (sj < 0) {
                    sj = lastj;
                    sbase = lastbase;
                }
                s_seg0 = 256 * (t * kSegPerThread + sj);
                s_base = sbase;
                s_target = target;
            }
            __syncthreads();
            if (t < kWave) {
                const int y = token_in_segment(s_seg0, s_base, s_target);
                if (lane == 0) a.out_tokens[(int64_t)b * (g + 1) + J] = y;
            }
            return;
        }
        __syncthreads();  // no residual mass: the chunk path below, with p
    } else {
        block_sum2(zp, zq, dscr);
        iZp = 1.0 / zp;
        iZq = qrow ? 1.0 / zq : 0.0;
    }

    // otherwise: locate the chunk holding u* Z (wave 0), then scan it in token order
    if (threadIdx.x < kWave) {
        double zr = 0.0;
        for (int cc = threadIdx.x; cc < a.rnchunk; cc += kWave) zr += fmax(0.0, rp[cc].a * iZp - rp[cc].b * iZq);
        zr = wave_sum(zr);
        const bool usep = !(zr > 0.0);
        const double target = s_uextra * (usep ? 1.0 : zr);
        int chunk;
        double cbase;
        wave_find_chunk(a.rnchunk, target,
                        [&](int cc) { return usep ? rp[cc].wp * iZp : fmax(0.0, rp[cc].a * iZp - rp[cc].b * iZq); },
                        chunk, cbase);
        if (threadIdx.x == 0) {
            s_chunk = chunk;
            s_base = cbase;
            s_target = target;
            s_usep = usep;
        }
    }
    __syncthreads();
    const int cs = s_chunk;
    const bool usep = s_usep != 0;
    const int cbase = cs * kChunk;
    if (VEC && !(usep && qrow)) {
        // The residual (or p, with no draft row) has its segment sums stored: wave 0 finds the
        // segment holding u* Z, then the token inside it.
        if (threadIdx.x < kWave) {
            const int lane = threadIdx.x;
            const double target = s_target;
            const double *sg = w.seg + 2 * (((int64_t)b * a.rnchunk + cs) * kPerThread);
            const double v = lane < kPerThread ? fmax(0.0, sg[2 * lane] * iZp - sg[2 * lane + 1] * iZq) : 0.0;
            const double incl = wave_scan_incl(v, 0.0, OpAdd());
            const double excl = s_base + incl - v;
            const uint64_t pass = __ballot(v > 0.0 && s_base + incl > target);
            const uint64_t posm = __ballot(v > 0.0);
            // rounding can leave every running sum at or below target: the last segment with mass
            const int sseg = pass ? __ffsll((unsigned long long)pass) - 1
                                  : (posm ? 63 - __clzll((unsigned long long)posm) : 0);
            const int y = token_in_segment(cbase + 256 * sseg, lane_value(excl, sseg), target);
            if (lane == 0) a.out_tokens[(int64_t)b * (g + 1) + J] = y;
        }
        return;
    }
    const bool twor = !usep && qrow;
    auto weight = [&](float lp, float lq) -> double { return twor ? r_of(lp, lq) : wp_of(lp) * iZp; };
    int y = chunk_inverse_cdf<PER, VEC>(prow, twor ? qrow : nullptr, cbase, a.V, s_base, s_target, weight, scan, iscr);
    if (y < 0) y = cbase;  // no mass in the chunk at all (cannot happen for the chunk found)
    if (threadIdx.x == 0) a.out_tokens[(int64_t)b * (g + 1) + J] = y;
}

// ---------------------------------------------------------------------------
// Block verification ("Speculative Decoding: The Art of Guessing Well", section "Block
// verification"), after the statistics pass:
//   block pass  grid (4096-token chunk, candidate k = 0..gamma, sequence).  Candidate k
//               keeps k drafts; its residual (w_k p_{k+1} - q_{k+1})+ lives on target row
//               k and draft row k (none for k = gamma).  Every block weighs its chunk of
//               both rows in fp64 (exp2_acc) and stores the sums of wp and wq over every
//               token, and (A, B) = the sums over the tokens whose residual is positive by
//               the statistics pass's estimates (normalizers and w_k), per chunk and per
//               256-token segment.
//   decide      one block per sequence: exact normalizers (sums of the chunk totals), exact
//               p_k(x_k), q_k(x_k) and running weights w_k, masses m_k = sum over chunks of
//               max(0, w_k A/Zp - B/Zq) (m_gamma = w_gamma), survival h_k =
//               m_k / (m_k + 1 - w_k), n = the longest prefix with u_{k-1} <= h_k, then the
//               draw from candidate n's segments as in the residual draw.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double next_weight(double w, double p, double q)
{
    return q > 0.0 ? fmin(1.0, w * p / q) : ((w > 0.0 && p > 0.0) ? 1.0 : 0.0);
}

template <bool VEC>
__global__ __launch_bounds__(kRowThreads, 2) void accept_block_pass_kernel(AcceptArgs a, AcceptWs w)
{
    constexpr int PER = kBlockPer;
    extern __shared__ __align__(16) unsigned char dyn_lds[];
    __shared__ double sM[129], sZ[129];
    __shared__ double dscr[2 * (kRowThreads / kWave)];
    __shared__ double s_p[64], s_q[64];
    __shared__ double s_w;
    const int c = blockIdx.x, kc = blockIdx.y, b = blockIdx.z;
    const int g = a.gamma;
    const int gb = gamma_of(a, b);
    if (kc > gb) return;  // a candidate past the sequence's length
    const int nch = gridDim.x;
    // the drafted tokens' logits (estimates of p_j(x_j), q_j(x_j) for j < kc)
    const int ti = min((int)threadIdx.x, g - 1);
    const int x = a.tokens[(int64_t)b * g + ti];
    const int xc = min(max(x, 0), a.V - 1);
    const float lpx = a.target[((int64_t)b * (g + 1) + ti) * a.V + xc];
    const float lqx = a.draft[((int64_t)b * g + ti) * a.V + xc];
    const RowPart *pp = w.part + (int64_t)b * a.rows * a.npart;
    RowPart *stage = reinterpret_cast<RowPart *>(dyn_lds);
    if (a.rows * a.npart <= kMaxStaged) {
        stage_parts(pp, a.rows * a.npart, stage, [] {});
        row_softmax_stats(stage, a.rows, a.npart, a.kd, sM, sZ);
    } else {
        row_softmax_stats(pp, a.rows, a.npart, a.kd, sM, sZ);
    }
    if ((int)threadIdx.x < kc) {
        const int j = threadIdx.x;
        s_p[j] = exp(((double)lpx - sM[j]) * a.inv_t) / sZ[j];
        s_q[j] = exp(((double)lqx - sM[g + 1 + j]) * a.inv_t) / sZ[g + 1 + j];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double wk = 1.0;
        for (int j = 0; j < kc; ++j) wk = next_weight(wk, s_p[j], s_q[j]);
        s_w = wk;
    }
    __syncthreads();
    const double wk = s_w;
    const float *prow = a.target + ((int64_t)b * (g + 1) + kc) * a.V;
    const float *qrow = kc < gb ? a.draft + ((int64_t)b * g + kc) * a.V : prow;
    const double Mp = sM[kc], Mq = kc < gb ? sM[g + 1 + kc] : Mp;
    const double nMpk = -Mp * a.kd, nMqk = -Mq * a.kd;  // exponents as one multiply-add each
    const double iZp_est = 1.0 / sZ[kc], iZq_est = kc < gb ? 1.0 / sZ[g + 1 + kc] : 0.0;
    const double qmask = kc < gb ? 1.0 : 0.0;
    float xp[PER], xq[PER];
    load_chunk2<VEC, PER>(prow, qrow, c * kBlockChunk, a.V, xp, xq);
    double ta = 0.0, tb = 0.0, tp = 0.0, tq = 0.0;
    double a4[PER / 4], b4[PER / 4];
#pragma unroll
    for (int k4 = 0; k4 < PER / 4; ++k4) {
        a4[k4] = 0.0;
        b4[k4] = 0.0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const double wp = exp2_acc(fma((double)xp[4 * k4 + j], a.kd, nMpk));
            const double wq = exp2_acc(fma((double)xq[4 * k4 + j], a.kd, nMqk)) * qmask;
            tp += wp;
            tq += wq;
            const bool in = wk * wp * iZp_est > wq * iZq_est;
            a4[k4] += in ? wp : 0.0;
            b4[k4] += in ? wq : 0.0;
        }
        ta += a4[k4];
        tb += b4[k4];
    }
    const int64_t slot = ((int64_t)b * (g + 1) + kc) * nch + c;
    if (VEC) {
        const int wv = threadIdx.x / kWave;
        double *sg = w.bseg + slot * PER * 2;
#pragma unroll
        for (int k4 = 0; k4 < PER / 4; ++k4) {
            const double sa = wave_sum(a4[k4]), sb = wave_sum(b4[k4]);
            if (threadIdx.x % kWave == 0) {
                sg[2 * (4 * k4 + wv)] = sa;
                sg[2 * (4 * k4 + wv) + 1] = sb;
            }
        }
    }
    block_sum2(ta, tb, dscr);
    block_sum2(tp, tq, dscr);
    if (threadIdx.x == 0) w.bchunk[slot] = BlockChunk{ta, tb, tp, tq};
}

// One-pass draw over per-segment masses held kSegPerThread to a thread, in token order:
// finds the segment whose running mass passes target = u * (the total); when rounding
// leaves every running sum at or below target, the last segment with mass.  Returns
// false (in every thread) when the total is not positive; else s_seg, s_base (the mass
// before the segment) and s_target are set for the whole block.
__device__ bool draw_segment(const double (&v)[kSegPerThread], double u, double *dscr, int *s_whit, int *s_wlast,
                             int *s_seg, double *s_base, double *s_target)
{
    const int t = threadIdx.x, lane = t % kWave, wv = t / kWave;
    const double ts = ((v[0] + v[1]) + v[2]) + v[3];
    const double incl_w = wave_scan_incl(ts, 0.0, OpAdd());
    __syncthreads();
    if (lane == kWave - 1) dscr[wv] = incl_w;
    __syncthreads();
    double wbase = 0.0, zr = 0.0;
#pragma unroll
    for (int k = 0; k < kRowThreads / kWave; ++k) {
        if (k < wv) wbase += dscr[k];
        zr += dscr[k];
    }
    if (!(zr > 0.0)) return false;
    const double incl = wbase + incl_w;
    const double target = u * zr;
    const uint64_t hit = __ballot(ts > 0.0 && incl > target);
    const uint64_t pos = __ballot(ts > 0.0);
    if (lane == 0) {
        s_whit[wv] = hit ? wv * kWave + __ffsll((unsigned long long)hit) - 1 : kRowThreads;
        s_wlast[wv] = pos ? wv * kWave + 63 - __clzll((unsigned long long)pos) : -1;
    }
    __syncthreads();
    int th = kRowThreads, tl = -1;
#pragma unroll
    for (int k = 0; k < kRowThreads / kWave; ++k) {
        th = min(th, s_whit[k]);
        tl = max(tl, s_wlast[k]);
    }
    if (t == (th < kRowThreads ? th : tl)) {
        double cum = incl - ts;
        int sj = -1, lastj = 0;
        double sbase = cum, lastbase = cum;
#pragma unroll
        for (int j = 0; j < kSegPerThread; ++j) {
            if (v[j] > 0.0) {
                if (sj < 0 && cum + v[j] > target) {
                    sj = j;
                    sbase = cum;
                }
                lastj = j;
                lastbase = cum;
            }
            cum += v[j];
        }
        if (sj < 0) {
            sj = lastj;
            sbase = lastbase;
        }
        *s_seg = t * kSegPerThread + sj;
        *s_base = sbase;
        *s_target = target;
    }
    __syncthreads();
    return true;
}

// One wave: the token of the 256-token segment starting at seg0 whose running weight, from
// sbase, passes target (weights r(l_p, l_q) of four tokens per lane); the last token with
// weight when rounding stops short.  Every lane returns it.
template <typename W>
__device__ int wave_token_in_segment(const float *prow, const float *qrow, int V, int seg0, double sbase,
                                     double target, W r)
{
    const int lane = threadIdx.x % kWave;
    const int e0 = seg0 + 4 * lane;
    double wt[4];
    if (V % 4 == 0) {
        const int ec = min(e0, V - 4);
        const float4 fp = *reinterpret_cast<const float4 *>(prow + ec);
        const float4 fq = *reinterpret_cast<const float4 *>(qrow + ec);
        const bool in = e0 < V;
        wt[0] = in ? r(fp.x, fq.x) : 0.0;
        wt[1] = in ? r(fp.y, fq.y) : 0.0;
        wt[2] = in ? r(fp.z, fq.z) : 0.0;
        wt[3] = in ? r(fp.w, fq.w) : 0.0;
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = min(e0 + j, V - 1);
            wt[j] = e0 + j < V ? r(prow[e], qrow[e]) : 0.0;
        }
    }
    const double lsum = ((wt[0] + wt[1]) + wt[2]) + wt[3];
    const double c0 = sbase + wave_scan_incl(lsum, 0.0, OpAdd()) - lsum;
    int hit = -1, lastpos = -1;
    double pre = c0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        pre += wt[j];
        if (hit < 0 && pre > target && wt[j] > 0.0) hit = j;
        if (wt[j] > 0.0) lastpos = j;
    }
    const uint64_t hm = __ballot(c0 <= target && hit >= 0);
    const uint64_t lm = __ballot(lastpos >= 0);
    if (hm) {
        const int hl = __ffsll((unsigned long long)hm) - 1;
        return seg0 + 4 * hl + lane_value(hit, hl);
    }
    if (lm) {
        const int ll = 63 - __clzll((unsigned long long)lm);
        return seg0 + 4 * ll + lane_value(lastpos, ll);
    }
    return seg0;
}

template <bool VEC>
__global__ __launch_bounds__(kRowThreads) void accept_block_decide_kernel(AcceptArgs a, AcceptWs w, int nch)
{
    extern __shared__ __align__(16) unsigned char dyn_lds[];
    __shared__ double sM[129], sZ[129];
    __shared__ double dscr[2 * (kRowThreads / kWave)];
    __shared__ double s_zp[65], s_zq[65], s_m[65], s_wt[65], s_p[64], s_q[64];
    __shared__ double s_base, s_target, s_ustar;
    __shared__ int s_n, s_seg, s_chunk, s_usep, bad;
    __shared__ int s_whit[kRowThreads / kWave], s_wlast[kRowThreads / kWave];
    __shared__ double scan[kRowThreads];
    __shared__ int iscr[kRowThreads / kWave];
    const int b = blockIdx.x;
    const int g = a.gamma;
    const int gb = gamma_of(a, b);  // this sequence's drafts: candidates 0..gb
    const int ti = min((int)threadIdx.x, g - 1);
    const int x = a.tokens[(int64_t)b * g + ti];
    const int xc = min(max(x, 0), a.V - 1);
    const float lpx = a.target[((int64_t)b * (g + 1) + ti) * a.V + xc];
    const float lqx = a.draft[((int64_t)b * g + ti) * a.V + xc];
    const double u_mine = w.u[(int64_t)b * (g + 1) + min((int)threadIdx.x, g)];
    if (threadIdx.x == 0) bad = 0;
    const RowPart *pp = w.part + (int64_t)b * a.rows * a.npart;
    RowPart *stage = reinterpret_cast<RowPart *>(dyn_lds);
    if (a.rows * a.npart <= kMaxStaged) {
        stage_parts(pp, a.rows * a.npart, stage, [] {});
        row_softmax_stats(stage, a.rows, a.npart, a.kd, sM, sZ);
    } else {
        row_softmax_stats(pp, a.rows, a.npart, a.kd, sM, sZ);
    }
    // exact normalizers of every candidate's rows, and the masses' (A, B) sums: one wave per
    // candidate, lanes over the chunks, fixed order
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const BlockChunk *bc = w.bchunk + (int64_t)b * (g + 1) * nch;
    for (int kc = wave; kc <= gb; kc += kRowThreads / kWave) {
        double zp = 0.0, zq = 0.0;
        for (int c = lane; c < nch; c += kWave) {
            zp += bc[(int64_t)kc * nch + c].wp;
            zq += bc[(int64_t)kc * nch + c].wq;
        }
        zp = wave_sum(zp);
        zq = wave_sum(zq);
        if (lane == 0) {
            s_zp[kc] = zp;
            s_zq[kc] = zq;
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < gb) {
        const int j = threadIdx.x;
        s_p[j] = exp2_acc(((double)lpx - sM[j]) * a.kd) / s_zp[j];
        s_q[j] = exp2_acc(((double)lqx - sM[g + 1 + j]) * a.kd) / s_zq[j];
        if (x < 0 || x >= a.V) bad = 1;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        s_wt[0] = 1.0;
        for (int k = 1; k <= gb; ++k) s_wt[k] = next_weight(s_wt[k - 1], s_p[k - 1], s_q[k - 1]);
    }
    __syncthreads();
    for (int kc = wave; kc <= gb; kc += kRowThreads / kWave) {
        const double wk = s_wt[kc], ip = 1.0 / s_zp[kc], iq = kc < gb ? 1.0 / s_zq[kc] : 0.0;
        double m = 0.0;
        for (int c = lane; c < nch; c += kWave) {
            const BlockChunk q = bc[(int64_t)kc * nch + c];
            m += fmax(0.0, wk * q.a * ip - q.b * iq);
        }
        m = wave_sum(m);
        if (lane == 0) s_m[kc] = kc < gb ? m : s_wt[gb];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int n = 0;
        for (int k = 1; k <= gb; ++k) {
            const double wk = s_wt[k], mk = s_m[k];
            const double h = wk < 1.0 ? mk / (mk + 1.0 - wk) : 1.0;
            // the survival uniforms are w.u[b][0..gb-1], the draw's w.u[b][gb]
            if (w.u[(int64_t)b * (g + 1) + k - 1] <= h) n = k;
        }
        s_n = n;
    }
    __syncthreads();
    const int n = s_n;
    int32_t *out = a.out_tokens + (int64_t)b * (g + 1);
    for (int i = threadIdx.x; i <= g; i += kRowThreads)
        if (i != n) out[i] = i < n ? a.tokens[(int64_t)b * g + i] : -1;
    if (threadIdx.x == 0) {
        a.accept_len[b] = n;
        if (a.dev_status) a.dev_status[b] = status_of(a, b, bad);
    }
    // the draw from (w_n p_{n+1} - q_{n+1})+ (candidate n), with the uniform thread gb holds
    if ((int)threadIdx.x == gb) s_ustar = u_mine;
    __syncthreads();
    const double us = s_ustar;
    const float *prow = a.target + ((int64_t)b * (g + 1) + n) * a.V;
    const float *qrow = n < gb ? a.draft + ((int64_t)b * g + n) * a.V : prow;
    const double Mp = sM[n], Mq = n < gb ? sM[g + 1 + n] : Mp;
    const double wn = s_wt[n], ip = 1.0 / s_zp[n], iq = n < gb ? 1.0 / s_zq[n] : 0.0;
    const double qmask = n < gb ? 1.0 : 0.0;
    auto r_of = [&](float lp, float lq) {
        return fmax(0.0, wn * exp2_acc(((double)lp - Mp) * a.kd) * ip -
                             exp2_acc(((double)lq - Mq) * a.kd) * qmask * iq);
    };
    const int nseg = nch * kBlockPer;
    if (VEC && nseg <= kRowThreads * kSegPerThread) {
        const int t = threadIdx.x;
        const bool live = t * kSegPerThread < nseg;
        const double2 *sg = reinterpret_cast<const double2 *>(
            w.bseg + (((int64_t)b * (g + 1) + n) * nch) * kBlockPer * 2 +
            (int64_t)min(t, nseg / kSegPerThread - 1) * kSegPerThread * 2);
        double v[kSegPerThread];
#pragma unroll
        for (int j = 0; j < kSegPerThread; ++j) {
            const double2 h = sg[j];
            v[j] = live ? fmax(0.0, wn * h.x * ip - h.y * iq) : 0.0;
        }
        if (draw_segment(v, us, dscr, s_whit, s_wlast, &s_seg, &s_base, &s_target)) {
            if (threadIdx.x < kWave) {
                const int y = wave_token_in_segment(prow, qrow, a.V, 256 * s_seg, s_base, s_target, r_of);
                if (lane == 0) out[n] = y;
            }
            return;
        }
    }
    // chunk path: the chunk holding u* Z (wave 0), then the token inside it (the block); a
    // residual without mass draws from p_{n+1}
    if (threadIdx.x < kWave) {
        const BlockChunk *q = bc + (int64_t)n * nch;
        double zr = 0.0;
        for (int c = lane; c < nch; c += kWave) zr += fmax(0.0, wn * q[c].a * ip - q[c].b * iq);
        zr = wave_sum(zr);
        const bool usep = !(zr > 0.0);
        const double target = us * (usep ? 1.0 : zr);
        int chunk;
        double cbase;
        wave_find_chunk(nch, target,
                        [&](int c) { return usep ? q[c].wp * ip : fmax(0.0, wn * q[c].a * ip - q[c].b * iq); },
                        chunk, cbase);
        if (lane == 0) {
            s_chunk = chunk;
            s_base = cbase;
            s_target = target;
            s_usep = usep;
        }
    }
    __syncthreads();
    const bool usep = s_usep != 0;
    auto weight = [&](float lp, float lq) -> double {
        return usep ? exp2_acc(((double)lp - Mp) * a.kd) * ip : r_of(lp, lq);
    };
    int y = chunk_inverse_cdf<kBlockPer, VEC>(prow, qrow, s_chunk * kBlockChunk, a.V, s_base, s_target, weight,
                                              scan, iscr);
    if (y < 0) y = s_chunk * kBlockChunk;
    if (threadIdx.x == 0) out[n] = y;
}

// ---------------------------------------------------------------------------
// Gumbel-coupled verification ("Speculative Decoding: The Art of Guessing Well", section
// "Sampling with shared noise"):
//   gumbel pass  grid (4096-token chunk, position i = 0..gamma, sequence): the chunk's best
//                score l/T - log(-log u) in fp64 (ties to the lowest token).  Every thread
//                holds four groups of four consecutive tokens, so each group takes one
//                Philox block (counter (x div 4, step, stream, tag + 2^32 i)).  Scores are
//                first estimated in fp32 (hardware log2); only tokens whose estimate lies
//                within a margin of the chunk's best estimate -- far wider than the
//                estimate's error, so the fp64 winner is always among them -- get the fp64
//                score, which alone decides.
//   decide       one block per sequence: y_i = the best over the chunks, J = the first
//                mismatch of the drafts, outputs.
// ---------------------------------------------------------------------------
// fp32 estimate of -log(u) for the uniform u = (2 (w >> 12) + 1) 2^-53 of Philox word w,
// relative error under 1e-5: log2 of u itself when u < 1/2; otherwise -log(1 - r) of
// r = 1 - u, which is formed exactly from the integer, through a short series for r <= 1/64
// (log2 of a number near 1 would lose the relative precision there).
__device__ __forceinline__ float neg_log_uniform_f32(uint64_t w)
{
    constexpr float kLn2f = 0.69314718055994530942f;
    const uint64_t n = 2 * (w >> 12) + 1;          // u = n 2^-53
    const bool low = n < (1ull << 52);             // u < 1/2
    const uint64_t k = low ? n : (1ull << 53) - n; // 2^53 u, or 2^53 (1 - u)
    const float x = fmaf((float)(uint32_t)(k >> 32), 0x1p32f, (float)(uint32_t)k) * 0x1p-53f;
    if (low) return -__builtin_amdgcn_logf(x) * kLn2f;
    if (x <= 0x1p-6f) return x * (1.f + x * (0.5f + x * (1.f / 3.f + x * 0.25f)));
    return -__builtin_amdgcn_logf(1.f - x) * kLn2f;
}

template <bool VEC>
__global__ __launch_bounds__(kRowThreads) void accept_gumbel_pass_kernel(AcceptArgs a, AcceptWs w)
{
    constexpr float kLn2f = 0.69314718055994530942f;
    __shared__ double s_s[kRowThreads / kWave];
    __shared__ int s_i[kRowThreads / kWave];
    __shared__ float s_m[kRowThreads / kWave];
    const int c = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
    if (i > gamma_of(a, b)) return;  // a position past the sequence's length
    const int nch = gridDim.x;
    const float *row = a.target + ((int64_t)b * (a.gamma + 1) + i) * a.V;
    const int base = c * kBlockChunk;
    const uint64_t stream = stream_of(a, b);
    const uint64_t tag = kTagGumbel + ((uint64_t)i << 32);
    float lg[kBlockPer];
#pragma unroll
    for (int k4 = 0; k4 < kBlockPer / 4; ++k4) {
        const int e = base + 4 * (int)threadIdx.x + 1024 * k4;
        if (VEC) {
            const float4 f = *reinterpret_cast<const float4 *>(row + min(e, a.V - 4));
            lg[4 * k4 + 0] = f.x;
            lg[4 * k4 + 1] = f.y;
            lg[4 * k4 + 2] = f.z;
            lg[4 * k4 + 3] = f.w;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) lg[4 * k4 + j] = row[min(e + j, a.V - 1)];
        }
    }
    // fp32 estimates: |error| < 1e-5 (1 + |l/T| + |g|) with |g| < 37, g the Gumbel term
    const float itau = (float)(1.0 / a.tau);
    float est[kBlockPer];
    float m = -INFINITY;
#pragma unroll
    for (int k4 = 0; k4 < kBlockPer / 4; ++k4) {
        const int e = base + 4 * (int)threadIdx.x + 1024 * k4;
        uint64_t ctr[4] = {(uint64_t)e >> 2, a.step, stream, tag};
        if (e < a.V) philox4x64_10(ctr, a.seed, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            est[4 * k4 + j] = e + j < a.V
                                  ? lg[4 * k4 + j] * itau - __builtin_amdgcn_logf(neg_log_uniform_f32(ctr[j])) * kLn2f
                                  : -INFINITY;
            m = fmaxf(m, est[4 * k4 + j]);
        }
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    if (threadIdx.x % kWave == 0) s_m[threadIdx.x / kWave] = m;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kRowThreads / kWave; ++k) m = fmaxf(m, s_m[k]);
    // candidates: estimates within 1e-2 + 1e-3 |best| of the best estimate (a margin
    // hundreds of times the estimates' error).  When no estimate is above -inf, every
    // finite logit is a candidate (l/T can overflow fp32 while fp64 holds it).
    const float thr = m == INFINITY ? INFINITY : m - (1e-2f + 1e-3f * fabsf(m));
    const bool none = m == -INFINITY;
    unsigned cand = 0;
#pragma unroll
    for (int k4 = 0; k4 < kBlockPer / 4; ++k4) {
        const int e = base + 4 * (int)threadIdx.x + 1024 * k4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool in = none ? (e + j < a.V && lg[4 * k4 + j] > -INFINITY) : est[4 * k4 + j] >= thr;
            cand |= (unsigned)in << (4 * k4 + j);
        }
    }
    // exact fp64 scores of the candidates, in increasing token order (ties keep the first)
    double best = -INFINITY;
    int arg = 0x7fffffff;
    while (cand) {
        const int j = __builtin_ctz(cand);
        cand &= cand - 1;
        const int e = base + 4 * (int)threadIdx.x + 1024 * (j >> 2) + (j & 3);
        uint64_t ctr[4] = {(uint64_t)e >> 2, a.step, stream, tag};
        philox4x64_10(ctr, a.seed, 0);
        const uint64_t wj = (j & 3) == 0 ? ctr[0] : (j & 3) == 1 ? ctr[1] : (j & 3) == 2 ? ctr[2] : ctr[3];
        const double u = (double)(2 * (wj >> 12) + 1) * 0x1p-53;
        const double sc = (double)row[e] / a.tau + (-log(-log(u)));
        if (sc > best) {
            best = sc;
            arg = e;
        }
    }
    // block argmax (larger score, then lower token)
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const double ob = __shfl_xor(best, off, kWave);
        const int oa = __shfl_xor(arg, off, kWave);
        if (ob > best || (ob == best && oa < arg)) {
            best = ob;
            arg = oa;
        }
    }
    const int wv = threadIdx.x / kWave;
    if (threadIdx.x % kWave == 0) {
        s_s[wv] = best;
        s_i[wv] = arg;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int k = 1; k < kRowThreads / kWave; ++k)
            if (s_s[k] > best || (s_s[k] == best && s_i[k] < arg)) {
                best = s_s[k];
                arg = s_i[k];
            }
        w.gpart[((int64_t)b * (a.gamma + 1) + i) * nch + c] = GumbelPart{best, arg, 0};
    }
}

__global__ __launch_bounds__(kRowThreads) void accept_gumbel_decide_kernel(AcceptArgs a, AcceptWs w, int nch)
{
    __shared__ int y[65];
    __shared__ int firstbad, bad;
    const int b = blockIdx.x;
    const int g = a.gamma;
    const int gb = gamma_of(a, b);
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    if (threadIdx.x == 0) {
        firstbad = gb;
        bad = 0;
    }
    const GumbelPart *gp = w.gpart + (int64_t)b * (g + 1) * nch;
    for (int i = wave; i <= gb; i += kRowThreads / kWave) {
        double best = -INFINITY;
        int arg = 0x7fffffff;
        for (int c = lane; c < nch; c += kWave) {
            const GumbelPart q = gp[(int64_t)i * nch + c];
            if (q.s > best || (q.s == best && q.arg < arg)) {
                best = q.s;
                arg = q.arg;
            }
        }
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const double ob = __shfl_xor(best, off, kWave);
            const int oa = __shfl_xor(arg, off, kWave);
            if (ob > best || (ob == best && oa < arg)) {
                best = ob;
                arg = oa;
            }
        }
        if (lane == 0) y[i] = arg;
    }
    __syncthreads();
    if ((int)threadIdx.x < gb) {
        const int x = a.tokens[(int64_t)b * g + threadIdx.x];
        if (x != y[threadIdx.x]) atomicMin(&firstbad, (int)threadIdx.x);
        if (x < 0 || x >= a.V) bad = 1;
    }
    __syncthreads();
    const int J = firstbad;
    int32_t *out = a.out_tokens + (int64_t)b * (g + 1);
    for (int i = threadIdx.x; i <= g; i += kRowThreads) out[i] = i < J ? a.tokens[(int64_t)b * g + i] : (i == J ? y[J] : -1);
    if (a.alpha)
        for (int i = threadIdx.x; i < g; i += kRowThreads) a.alpha[(int64_t)b * g + i] = __int_as_float(0x7fc00000);
    if (threadIdx.x == 0) {
        a.accept_len[b] = J;
        if (a.dev_status) a.dev_status[b] = status_of(a, b, bad);
    }
}

template <typename K>
static hipError_t launch(K kernel, dim3 grid, hipStream_t s, const AcceptArgs &a, const AcceptWs &w, size_t lds = 0)
{
    hipLaunchKernelGGL(kernel, grid, dim3(kRowThreads), lds, s, a, w);
    return hipGetLastError();
}

// Blocks of a looping kernel that are resident at once on the current device (occupancy
// x compute units), asked of the runtime on every call.
template <bool VEC, bool SAMPLE, int PER>
static int stats_resident_blocks()
{
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, accept_stats_kernel<VEC, SAMPLE, PER>, kRowThreads, 0) !=
            hipSuccess ||
        per_cu < 1)
        per_cu = 2;
    return per_cu * device_cu_count();
}

// The residual draw runs on chunks of its own: kResChunk (2048) tokens for small calls in
// the vector layout, 4096 otherwise.  Each of its tokens takes two fp64 exponentials, so
// the statistics pass's 16384-token chunks would hold 128 logits per thread (256 registers
// and spills, 50 us on the 64-sequence batch).
template <bool VEC, int PER>
static hipError_t launch_resample(const AcceptArgs &a0, const AcceptWs &w, hipStream_t s, size_t lds)
{
    AcceptArgs a = a0;
    constexpr int RP = (VEC && PER == 16) ? kResPer : 16;
    a.rnchunk = (a.V + RP * kRowThreads - 1) / (RP * kRowThreads);
    // Blocks per sequence: as many as fit on the GPU at once, at most one per chunk.  On the
    // 64-sequence batch (32 chunks per sequence), a block per chunk took 84 us per call, the
    // resident grid 76 (its next chunk prefetched meanwhile: no better).
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, accept_resample_kernel<VEC, RP>, kRowThreads, lds) !=
            hipSuccess || per_cu < 1)
        per_cu = 2;
    const int64_t resident = (int64_t)per_cu * device_cu_count();
    const int64_t per_seq = resident / a.B;
    const int gx = (int)(per_seq >= a.rnchunk ? a.rnchunk : per_seq < 1 ? 1 : per_seq);
    return launch(accept_resample_kernel<VEC, RP>, dim3(gx, a.B), s, a, w, lds);
}

template <bool VEC, int PER>
static sv_status run_accept(const AcceptArgs &a, const AcceptWs &w, hipStream_t s, bool sample, bool alpha)
{
    // staging slots: the part count rounded up to 1, 2, 4 or 8 per thread
    const int staged = a.rows * a.npart;
    int slots = kRowThreads;
    while (slots < staged) slots *= 2;
    const size_t lds = staged <= kMaxStaged ? (size_t)slots * sizeof(RowPart) : 0;
    const int64_t ntask = (int64_t)a.nchunk * (a.rows + (sample ? 1 : 0)) * a.B;
    const int64_t resident = sample ? stats_resident_blocks<VEC, true, PER>() : stats_resident_blocks<VEC, false, PER>();
    // up to four rounds of resident blocks, one task each; larger calls loop over tasks
    // (64-sequence batch, 5120 tasks: grids of 1, 2, 3, 4 rounds 77.5, 76.9, 75.8, 74.5 us;
    // 6 and 8 rounds 74.8 and 74.6 us)
    const int64_t cap = 4 * resident;
    const dim3 gstats((unsigned)(ntask < cap ? ntask : cap));
    if (!sample) {
        if (launch(accept_stats_kernel<VEC, false, PER>, gstats, s, a, w) != hipSuccess) return SV_ERR_HIP;
        return launch(accept_greedy_kernel, dim3(a.B), s, a, w, lds) == hipSuccess ? SV_OK : SV_ERR_HIP;
    }
    const int bnch = (a.V + kBlockChunk - 1) / kBlockChunk;
    if (a.rule == SV_RULE_GUMBEL) {  // no statistics: Gumbel scores need no normalizer
        if (launch(accept_gumbel_pass_kernel<VEC>, dim3(bnch, a.gamma + 1, a.B), s, a, w) != hipSuccess)
            return SV_ERR_HIP;
        hipLaunchKernelGGL(accept_gumbel_decide_kernel, dim3(a.B), dim3(kRowThreads), 0, s, a, w, bnch);
        return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
    }
    if (launch(accept_stats_kernel<VEC, true, PER>, gstats, s, a, w) != hipSuccess) return SV_ERR_HIP;
    if (alpha && launch(accept_alpha_kernel<VEC, PER>, dim3(a.nchunk, a.gamma, a.B), s, a, w) != hipSuccess)
        return SV_ERR_HIP;
    if (a.rule == SV_RULE_BLOCK) {
        if (launch(accept_block_pass_kernel<VEC>, dim3(bnch, a.gamma + 1, a.B), s, a, w, lds) != hipSuccess)
            return SV_ERR_HIP;
        hipLaunchKernelGGL(accept_block_decide_kernel<VEC>, dim3(a.B), dim3(kRowThreads), lds, s, a, w, bnch);
        return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
    }
    return launch_resample<VEC, PER>(a, w, s, lds) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // namespace

extern "C" size_t sv_spec_accept_workspace(const sv_accept_desc *d)
{
    if (!d || d->B < 0 || d->gamma < 1 || d->V < 1) return 0;
    if (d->rule != SV_RULE_TOKEN && d->rule != SV_RULE_BLOCK && d->rule != SV_RULE_GUMBEL) return 0;
    return accept_layout(d->B, d->gamma, d->V, d->rule).total;
}

extern "C" sv_status sv_spec_accept(const sv_accept_desc *d, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!d) return SV_ERR_INVALID_ARG;
    if (d->B < 0 || d->gamma < 1 || d->V < 1) return SV_ERR_INVALID_ARG;
    if (d->mode != SV_GREEDY && d->mode != SV_SAMPLE) return SV_ERR_INVALID_ARG;
    if (!(d->temperature >= 0.0f) || d->temperature == INFINITY) return SV_ERR_INVALID_ARG;
    if (d->gamma > 64) return SV_ERR_UNSUPPORTED;
    if (d->rule != SV_RULE_TOKEN && d->rule != SV_RULE_BLOCK && d->rule != SV_RULE_GUMBEL) return SV_ERR_INVALID_ARG;
    const bool sample = d->mode == SV_SAMPLE && d->temperature > 0.0f;
    if (!d->target_logits || !d->draft_tokens || !d->accept_len || !d->out_tokens) return SV_ERR_INVALID_ARG;
    if (sample && d->rule != SV_RULE_GUMBEL && !d->draft_logits) return SV_ERR_INVALID_ARG;
    if (d->B == 0) return SV_OK;
    if (d->B > kMaxCounters) return SV_ERR_UNSUPPORTED;
    const WsLayout L = accept_layout(d->B, d->gamma, d->V, d->rule);
    if (!workspace || workspace_bytes < L.total || ((uintptr_t)workspace & 255)) return SV_ERR_WORKSPACE;

    char *ws = (char *)workspace;
    AcceptWs w;
    w.cnt = (int *)(ws + L.cnt);
    w.part = (RowPart *)(ws + L.part);
    w.u = (double *)(ws + L.u);
    w.res = (ResPart *)(ws + L.res);
    w.seg = (double *)(ws + L.seg);
    w.apart = (double *)(ws + L.apart);
    w.bchunk = (BlockChunk *)(ws + L.bchunk);
    w.bseg = (double *)(ws + L.bseg);
    w.gpart = (GumbelPart *)(ws + L.gchunk);

    AcceptArgs a;
    a.B = d->B;
    a.gamma = d->gamma;
    a.V = d->V;
    a.rows = sample ? 2 * d->gamma + 1 : d->gamma + 1;
    a.sample = sample;
    const double T = sample ? (double)d->temperature : 1.0;
    a.kd = 1.4426950408889634 / T;
    a.kf = (float)a.kd;
    a.inv_t = 1.0 / T;
    a.tau = T;
    a.rule = d->rule;
    a.target = d->target_logits;
    a.draft = d->draft_logits;
    a.tokens = d->draft_tokens;
    a.seed = d->rng.seed;
    a.step = d->rng.step;
    a.stream_ids = d->rng.stream_ids;
    a.accept_len = d->accept_len;
    a.out_tokens = d->out_tokens;
    a.dev_status = d->dev_status;
    a.alpha = d->alpha;
    a.draft_len = d->draft_len;

    const bool vec = (d->V % 4 == 0) && (((uintptr_t)d->target_logits & 15) == 0) &&
                     (!sample || ((uintptr_t)d->draft_logits & 15) == 0);
    const int big_chunks = (d->V + 4 * kMinChunk - 1) / (4 * kMinChunk);
    // (threshold measured: calls of 704 and 896 big chunks ran 9-21% faster on the large
    // chunks, calls of 544 up to 15% slower)
    const bool wide = (int64_t)a.B * a.rows * big_chunks >= 640;
    a.nchunk = wide ? big_chunks : (d->V + kMinChunk - 1) / kMinChunk;
    a.npart = a.nchunk * (wide ? parts_per_chunk<64>() : parts_per_chunk<16>());
    a.rnchunk = a.nchunk;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    return wide ? (vec ? run_accept<true, 64>(a, w, s, sample, d->alpha != nullptr)
                       : run_accept<false, 64>(a, w, s, sample, d->alpha != nullptr))
                : (vec ? run_accept<true, 16>(a, w, s, sample, d->alpha != nullptr)
                       : run_accept<false, 16>(a, w, s, sample, d->alpha != nullptr));
}

// ---------------------------------------------------------------------------
// Allocation-free variant: the workspace is `scratch`, a fixed device array of this file
// (one copy per GPU, held until the process ends).  In host code `scratch` names only a
// host-side stand-in, so its device address is asked of the runtime once per device (with
// that device current) and kept; kernels get that address, never the array's name.
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = (size_t)SV_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up
}  // namespace

static sv_status scratch_address(void **ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SV_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return SV_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SV_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return SV_OK;
}

extern "C" sv_status sv_spec_accept_static(const sv_accept_desc *d, void *stream)
{
    // the size check reads only B, gamma and V, and comes before any runtime call
    if (d && sv_spec_accept_workspace(d) > kStaticScratchBytes) return SV_ERR_WORKSPACE;
    void *ws = nullptr;
    const sv_status st = scratch_address(&ws);
    if (st != SV_OK) return st;
    // the kernels clear the counters they use (accept_stats_kernel), so whatever an earlier
    // call left in the array does no harm; calls that overlap in time on one GPU race
    return sv_spec_accept(d, ws, kStaticScratchBytes, stream);
}

