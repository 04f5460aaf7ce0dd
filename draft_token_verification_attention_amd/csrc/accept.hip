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
//   stats   grid (chunk, row, sequence).  Each block reads 4096 logits of one row once:
//           GREEDY keeps (max, first argmax); SAMPLE keeps (chunk max m_c, S_c =
//           sum exp((l - m_c)/T) in fp64).  The last block of a sequence combines the
//           row statistics, draws the ratio-test uniforms and decides J (and, under
//           GREEDY, the extra token z_J).
//   alpha   optional: sum_x min(p_i, q_i) per draft position (one more read of the rows).
//   sample  SAMPLE only, grid (chunk, sequence): residual mass per chunk of the two rows
//           at position J; the last block finds the chunk holding u* Z and scans it in
//           token order for the extra token.
// Exponentials of the bulk run in fp32; every sum, the CDF and the decided p(x), q(x)
// are fp64.
#include "vocab_row.h"

namespace {

using namespace sv;

// A block reads 4096 (PER = 16) or 16384 (PER = 64) logits of one row, all loaded
// before any reduction: the larger chunk when the call has blocks to spare (big batches),
// the smaller one when latency matters (a single sequence).
constexpr int kMinChunk = 16 * kRowThreads;

struct RowPart {
    float m;
    int32_t arg;
    double s;
};
struct RowStat {
    double M;
    double Z;
};
struct SeqState {
    int32_t J;
    int32_t pad;
    double Mp, Zp, Mq, Zq;
};
struct ResPart {
    double r;
    double p;
};

struct AcceptWs {
    int *cnt;  // [B]: one completion counter per sequence, shared by the call's kernels in turn
    RowPart *part;      // [B][rows][nchunk]
    RowStat *rowstat;   // [B][rows]
    SeqState *seq;      // [B]
    ResPart *res;       // [B][nchunk]
    double *apart;      // [B][gamma][nchunk]
};

struct AcceptArgs {
    int B, gamma, V, rows, nchunk;
    int sample;
    float kf;          // log2(e) / T in fp32, for the bulk exponentials
    double inv_t;      // 1 / T in fp64, for decided probabilities
    double kd;         // log2(e) / T in fp64, for chunk rescaling
    const float *target, *draft;
    const int32_t *tokens;
    uint64_t seed, step;
    const uint64_t *stream_ids;
    int32_t *accept_len, *out_tokens, *dev_status;
    float *alpha;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
    size_t cnt, part, rowstat, seq, res, apart, total;
};

static WsLayout accept_layout(int B, int gamma, int V)
{
    const size_t rows = 2 * (size_t)gamma + 1;
    const size_t nchunk = ((size_t)V + kMinChunk - 1) / kMinChunk;  // the larger of the two chunk counts
    WsLayout L;
    size_t o = 0;
    L.cnt = o;
    o += kCounterBytes;
    L.part = o;
    o += align256((size_t)B * rows * nchunk * sizeof(RowPart));
    L.rowstat = o;
    o += align256((size_t)B * rows * sizeof(RowStat));
    L.seq = o;
    o += align256((size_t)B * sizeof(SeqState));
    L.res = o;
    o += align256((size_t)B * nchunk * sizeof(ResPart));
    L.apart = o;
    o += align256((size_t)B * gamma * nchunk * sizeof(double));
    L.total = o;
    return L;
}

__device__ __forceinline__ const float *row_ptr(const AcceptArgs &a, int b, int r)
{
    if (r <= a.gamma) return a.target + ((int64_t)b * (a.gamma + 1) + r) * a.V;
    return a.draft + ((int64_t)b * a.gamma + (r - a.gamma - 1)) * a.V;
}

__device__ __forceinline__ uint64_t stream_of(const AcceptArgs &a, int b)
{
    return a.stream_ids ? a.stream_ids[b] : (uint64_t)b;
}

// ---------------------------------------------------------------------------
// decide (runs in the last stats block of sequence b)
// ---------------------------------------------------------------------------
__device__ void decide_greedy(const AcceptArgs &a, const AcceptWs &w, int b)
{
    __shared__ int z[65];
    __shared__ int firstbad, bad;
    const int g = a.gamma;
    if (threadIdx.x == 0) {
        firstbad = g;
        bad = 0;
    }
    const int wave = threadIdx.x / kWave, nwaves = blockDim.x / kWave;
    for (int r = wave; r <= g; r += nwaves) {
        float v;
        int idx;
        wave_combine_argmax(w.part + ((int64_t)b * a.rows + r) * a.nchunk, a.nchunk, v, idx);
        if (threadIdx.x % kWave == 0) z[r] = idx;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < g; i += blockDim.x) {
        const int x = a.tokens[(int64_t)b * g + i];
        if (x != z[i]) atomicMin(&firstbad, i);
        if (x < 0 || x >= a.V) bad = 1;
    }
    __syncthreads();
    const int J = firstbad;
    int32_t *out = a.out_tokens + (int64_t)b * (g + 1);
    for (int i = threadIdx.x; i <= g; i += blockDim.x)
        out[i] = i < J ? a.tokens[(int64_t)b * g + i] : (i == J ? z[J] : -1);
    if (a.alpha)  // alpha is a sampling quantity
        for (int i = threadIdx.x; i < g; i += blockDim.x) a.alpha[(int64_t)b * g + i] = __int_as_float(0x7fc00000);
    if (threadIdx.x == 0) {
        a.accept_len[b] = J;
        if (a.dev_status) a.dev_status[b] = bad ? 2 : 0;
    }
}

__device__ void decide_sample(const AcceptArgs &a, const AcceptWs &w, int b)
{
    __shared__ double sM[129], sZ[129];
    __shared__ int firstbad, bad;
    const int g = a.gamma;
    if (threadIdx.x == 0) {
        firstbad = g;
        bad = 0;
    }
    const int wave = threadIdx.x / kWave, nwaves = blockDim.x / kWave;
    for (int r = wave; r < a.rows; r += nwaves) {
        float M;
        double Z;
        wave_combine_softmax(w.part + ((int64_t)b * a.rows + r) * a.nchunk, a.nchunk, a.kd, M, Z);
        if (threadIdx.x % kWave == 0) {
            sM[r] = (double)M;
            sZ[r] = Z;
            w.rowstat[(int64_t)b * a.rows + r] = RowStat{(double)M, Z};
        }
    }
    __syncthreads();
    const uint64_t stream = stream_of(a, b);
    for (int i = threadIdx.x; i < g; i += blockDim.x) {
        const int x = a.tokens[(int64_t)b * g + i];
        bool pass = false;
        if (x >= 0 && x < a.V) {
            const double lp = (double)a.target[((int64_t)b * (g + 1) + i) * a.V + x];
            const double lq = (double)a.draft[((int64_t)b * g + i) * a.V + x];
            const double p = exp((lp - sM[i]) * a.inv_t) / sZ[i];
            const double q = exp((lq - sM[g + 1 + i]) * a.inv_t) / sZ[g + 1 + i];
            const double u = philox_uniform(a.seed, (uint64_t)i, a.step, stream, kTagAccept);
            pass = u * q < p;
        } else {
            bad = 1;
        }
        if (!pass) atomicMin(&firstbad, i);
    }
    __syncthreads();
    const int J = firstbad;
    int32_t *out = a.out_tokens + (int64_t)b * (g + 1);
    for (int i = threadIdx.x; i <= g; i += blockDim.x) out[i] = i < J ? a.tokens[(int64_t)b * g + i] : -1;
    if (threadIdx.x == 0) {
        a.accept_len[b] = J;
        if (a.dev_status) a.dev_status[b] = bad ? 2 : 0;
        SeqState s;
        s.J = J;
        s.pad = 0;
        s.Mp = sM[J];
        s.Zp = sZ[J];
        s.Mq = J < g ? sM[g + 1 + J] : 0.0;
        s.Zq = J < g ? sZ[g + 1 + J] : 0.0;
        w.seq[b] = s;
    }
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
    __shared__ int last_flag;
    const int c = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
    const float *row = row_ptr(a, b, r);
    const int base = c * kChunk;
    float x[kPerThread];
    load_chunk<VEC, kPerThread>(row, base, a.V, x);

    RowPart part;
    if (!SAMPLE) {
        float v = -INFINITY;
        int idx = 0x7fffffff;
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
            const int e = chunk_index<VEC>(base, k);
            if (e < a.V) argmax_merge(v, idx, x[k], e);
        }
        block_argmax(v, idx, fscr, iscr);
        part.m = v;
        part.arg = idx;
        part.s = 0.0;
    } else {
        // each thread: its own max and its sum relative to it (no barrier); then the block
        // rescales the per-thread sums to the chunk max in fp64
        float mt = -INFINITY;
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) mt = fmaxf(mt, x[k]);
        double st = 0.0;
#pragma unroll
        for (int k = 0; k < kPerThread; ++k)
            if (x[k] != -INFINITY) st += (double)exp2f((x[k] - mt) * a.kf);
        const float m = block_max(mt, fscr);
        const double s = block_sum(st > 0.0 ? st * exp2(((double)mt - (double)m) * a.kd) : 0.0, dscr);
        part.m = m;
        part.arg = 0;
        part.s = s;
    }
    if (threadIdx.x == 0) {
        RowPart *dst = w.part + ((int64_t)b * a.rows + r) * a.nchunk + c;
        st_coherent(&dst->m, part.m);
        st_coherent(&dst->arg, part.arg);
        st_coherent(&dst->s, part.s);
    }
    if (!arrive_last(&w.cnt[b], a.rows * a.nchunk, &last_flag)) return;
    if (SAMPLE)
        decide_sample(a, w, b);
    else
        decide_greedy(a, w, b);
}

// ---------------------------------------------------------------------------
template <bool VEC, int PER>
__global__ __launch_bounds__(kRowThreads) void accept_alpha_kernel(AcceptArgs a, AcceptWs w)
{
    constexpr int kChunk = PER * kRowThreads;
    constexpr int kPerThread = PER;
    __shared__ double dscr[kRowThreads / kWave];
    __shared__ int last_flag;
    const int c = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
    const int g = a.gamma;
    const RowStat sp = w.rowstat[(int64_t)b * a.rows + i];
    const RowStat sq = w.rowstat[(int64_t)b * a.rows + g + 1 + i];
    const float Mp = (float)sp.M, Mq = (float)sq.M;
    const double iZp = 1.0 / sp.Z, iZq = 1.0 / sq.Z;
    float xp[kPerThread], xq[kPerThread];
    const int base = c * kChunk;
    load_chunk<VEC, kPerThread>(row_ptr(a, b, i), base, a.V, xp);
    load_chunk<VEC, kPerThread>(row_ptr(a, b, g + 1 + i), base, a.V, xq);
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        if (xp[k] == -INFINITY && xq[k] == -INFINITY) continue;
        const double p = (double)exp2f((xp[k] - Mp) * a.kf) * iZp;
        const double q = (double)exp2f((xq[k] - Mq) * a.kf) * iZq;
        s += fmin(p, q);
    }
    s = block_sum(s, dscr);
    if (threadIdx.x == 0) st_coherent(&w.apart[((int64_t)b * g + i) * a.nchunk + c], s);
    if (!arrive_last(&w.cnt[b], g * a.nchunk, &last_flag)) return;
    for (int j = threadIdx.x; j < g; j += blockDim.x) {
        double t = 0.0;
        for (int cc = 0; cc < a.nchunk; ++cc) t += w.apart[((int64_t)b * g + j) * a.nchunk + cc];
        a.alpha[(int64_t)b * g + j] = (float)t;
    }
}

// ---------------------------------------------------------------------------
template <bool VEC, int PER>
__global__ __launch_bounds__(kRowThreads) void accept_sample_kernel(AcceptArgs a, AcceptWs w)
{
    constexpr int kChunk = PER * kRowThreads;
    constexpr int kPerThread = PER;
    __shared__ double dscr[kRowThreads / kWave];
    __shared__ double scan[kRowThreads];
    __shared__ int iscr[kRowThreads / kWave];
    __shared__ int last_flag, s_chunk, s_usep;
    __shared__ double s_base, s_target;
    const int c = blockIdx.x, b = blockIdx.y;
    const int g = a.gamma;
    const SeqState st = w.seq[b];
    const int J = st.J;
    const float *prow = a.target + ((int64_t)b * (g + 1) + J) * a.V;
    const float *qrow = J < g ? a.draft + ((int64_t)b * g + J) * a.V : nullptr;
    const float Mp = (float)st.Mp, Mq = (float)st.Mq;
    const double iZp = 1.0 / st.Zp, iZq = J < g ? 1.0 / st.Zq : 0.0;
    const int base = c * kChunk;

    // weight of token e: residual (or p when every draft was kept / the residual is empty)
    auto p_of = [&](float l) { return (double)exp2f((l - Mp) * a.kf) * iZp; };
    auto q_of = [&](float l) { return (double)exp2f((l - Mq) * a.kf) * iZq; };

    float xp[kPerThread], xq[kPerThread];
    load_chunk<VEC, kPerThread>(prow, base, a.V, xp);
    if (qrow) load_chunk<VEC>(qrow, base, a.V, xq);
    double rs = 0.0, ps = 0.0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        if (xp[k] == -INFINITY) continue;
        const double p = p_of(xp[k]);
        ps += p;
        rs += qrow ? fmax(0.0, p - q_of(xq[k])) : p;
    }
    rs = block_sum(rs, dscr);
    ps = block_sum(ps, dscr);
    if (threadIdx.x == 0) {
        st_coherent(&w.res[(int64_t)b * a.nchunk + c].r, rs);
        st_coherent(&w.res[(int64_t)b * a.nchunk + c].p, ps);
    }
    if (!arrive_last(&w.cnt[b], a.nchunk, &last_flag)) return;

    // last block: locate the chunk holding u* Z (wave 0), then scan it in token order
    if (threadIdx.x < kWave) {
        const ResPart *rp = w.res + (int64_t)b * a.nchunk;
        double zr = 0.0, zp = 0.0;
        for (int cc = threadIdx.x; cc < a.nchunk; cc += kWave) {
            zr += rp[cc].r;
            zp += rp[cc].p;
        }
        zr = wave_sum(zr);
        zp = wave_sum(zp);
        const bool usep = !(zr > 0.0);
        const double u = philox_uniform(a.seed, (uint64_t)g, a.step, stream_of(a, b), kTagAccept);
        const double target = u * (usep ? zp : zr);
        int chunk;
        double cbase;
        wave_find_chunk(a.nchunk, target, [&](int cc) { return usep ? rp[cc].p : rp[cc].r; }, chunk, cbase);
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
    const bool twor = !usep && qrow;
    auto weight = [&](float lp, float lq) -> double {
        const double p = p_of(lp);
        return twor ? fmax(0.0, p - q_of(lq)) : p;
    };
    int y = chunk_inverse_cdf<PER, VEC>(prow, twor ? qrow : nullptr, cbase, a.V, s_base, s_target, weight, scan, iscr);
    if (y < 0) {
        // rounding left the running sum just short of u* Z: take the last token with mass
        int lastpos = -1;
        for (int e = cbase + (int)threadIdx.x; e < min(cbase + kChunk, a.V); e += kRowThreads)
            if (weight(prow[e], twor ? qrow[e] : prow[e]) > 0.0) lastpos = max(lastpos, e);
        y = block_max_int(lastpos, iscr);
        if (y < 0) y = cbase;
    }
    if (threadIdx.x == 0) a.out_tokens[(int64_t)b * (g + 1) + J] = y;
}

template <typename K>
static hipError_t launch(K kernel, dim3 grid, hipStream_t s, const AcceptArgs &a, const AcceptWs &w)
{
    hipLaunchKernelGGL(kernel, grid, dim3(kRowThreads), 0, s, a, w);
    return hipGetLastError();
}

template <bool VEC, int PER>
static sv_status run_accept(const AcceptArgs &a, const AcceptWs &w, hipStream_t s, bool sample, bool alpha)
{
    const dim3 gstats(a.nchunk, a.rows, a.B);
    if (!sample)
        return launch(accept_stats_kernel<VEC, false, PER>, gstats, s, a, w) == hipSuccess ? SV_OK : SV_ERR_HIP;
    if (launch(accept_stats_kernel<VEC, true, PER>, gstats, s, a, w) != hipSuccess) return SV_ERR_HIP;
    if (alpha && launch(accept_alpha_kernel<VEC, PER>, dim3(a.nchunk, a.gamma, a.B), s, a, w) != hipSuccess)
        return SV_ERR_HIP;
    return launch(accept_sample_kernel<VEC, PER>, dim3(a.nchunk, a.B), s, a, w) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // namespace

extern "C" size_t sv_spec_accept_workspace(const sv_accept_desc *d)
{
    if (!d || d->B < 0 || d->gamma < 1 || d->V < 1) return 0;
    return accept_layout(d->B, d->gamma, d->V).total;
}

extern "C" sv_status sv_spec_accept(const sv_accept_desc *d, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!d) return SV_ERR_INVALID_ARG;
    if (d->B < 0 || d->gamma < 1 || d->V < 1) return SV_ERR_INVALID_ARG;
    if (d->mode != SV_GREEDY && d->mode != SV_SAMPLE) return SV_ERR_INVALID_ARG;
    if (!(d->temperature >= 0.0f) || d->temperature == INFINITY) return SV_ERR_INVALID_ARG;
    if (d->gamma > 64) return SV_ERR_UNSUPPORTED;
    const bool sample = d->mode == SV_SAMPLE && d->temperature > 0.0f;
    if (!d->target_logits || !d->draft_tokens || !d->accept_len || !d->out_tokens) return SV_ERR_INVALID_ARG;
    if (sample && !d->draft_logits) return SV_ERR_INVALID_ARG;
    if (d->B == 0) return SV_OK;
    if (d->B > kMaxCounters) return SV_ERR_UNSUPPORTED;
    const WsLayout L = accept_layout(d->B, d->gamma, d->V);
    if (!workspace || workspace_bytes < L.total || ((uintptr_t)workspace & 255)) return SV_ERR_WORKSPACE;

    char *ws = (char *)workspace;
    AcceptWs w;
    w.cnt = (int *)(ws + L.cnt);
    w.part = (RowPart *)(ws + L.part);
    w.rowstat = (RowStat *)(ws + L.rowstat);
    w.seq = (SeqState *)(ws + L.seq);
    w.res = (ResPart *)(ws + L.res);
    w.apart = (double *)(ws + L.apart);

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

    const bool vec = (d->V % 4 == 0) && (((uintptr_t)d->target_logits & 15) == 0) &&
                     (!sample || ((uintptr_t)d->draft_logits & 15) == 0);
    const int big_chunks = (d->V + 4 * kMinChunk - 1) / (4 * kMinChunk);
    const bool wide = (int64_t)a.B * a.rows * big_chunks >= 1024;
    a.nchunk = wide ? big_chunks : (d->V + kMinChunk - 1) / kMinChunk;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    return wide ? (vec ? run_accept<true, 64>(a, w, s, sample, d->alpha != nullptr)
                       : run_accept<false, 64>(a, w, s, sample, d->alpha != nullptr))
                : (vec ? run_accept<true, 16>(a, w, s, sample, d->alpha != nullptr)
                       : run_accept<false, 16>(a, w, s, sample, d->alpha != nullptr));
}
