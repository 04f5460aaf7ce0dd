// commit.hip -- the KV-cache commit after a verification round.
//
// Sources: "Speculative decoding" (Zero to Frontier textbook, ch. 20, section 20.5),
// section "Keeping the caches consistent after a rejection": after J acceptances the
// entries of the accepted drafts are right and the rejected ones are discarded; a
// contiguous cache rolls back by moving its length pointer, and a tree needs one more step,
// gathering the accepted branch's entries (scattered among discarded siblings) into
// consecutive slots.  "Speculative Decoding: The Art of Guessing Well", section
// "Verification bottlenecks" (KV cache bookkeeping).
//
// One block per sequence.  The pass wrote node j at position P + j; path node k (k = 1..J)
// moves to P + k.  The moves run in path order in rounds: a round reads the K and V rows of
// its moves (all heads, 16-byte vectors in registers), waits for the whole block, then
// writes them.  A destination P + k never holds the source of a later move (path nodes
// satisfy node_k >= k and increase along the path), and a source overwritten by a later
// move was read in an earlier round, so the gather is safe in place.  The block then
// writes the new length P + 1 + J (it alone reads that sequence's length, so the output
// may be the length array itself).
#include "sv_common.h"

namespace {

using namespace sv;

constexpr int kCommitThreads = 256;
constexpr int kVecPerThread = 8;           // 16-byte vectors a thread holds per round
constexpr int kMaxPath = 65;               // path entries (the walk's max_depth <= 63, plus slack)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct CommitArgs {
    char *k, *v;
    const int64_t *kv_off;
    int64_t kv_sb, kv_sh, kv_st;  // elements
    int esize, B, n_q, Hkv, vpr;  // vpr: 16-byte vectors per row
    const int32_t *prefix_len, *accept_len, *path;
    int path_stride;
    int32_t *new_len, *dev_status;
};

__global__ __launch_bounds__(kCommitThreads) void kv_commit_kernel(CommitArgs a)
{
    __shared__ int s_node[kMaxPath];
    __shared__ int s_move[kMaxPath];
    __shared__ int s_bad, s_moves;
    const int b = blockIdx.x;
    const int t = threadIdx.x;
    const int P = a.prefix_len[b];
    const int J = a.accept_len[b];
    if (t == 0) {
        s_bad = !(J >= 0 && J < a.n_q && P >= 0 && (!a.path || J < a.path_stride));
        s_moves = 0;
    }
    __syncthreads();
    if (a.path && !s_bad && t >= 1 && t <= J) {
        const int node = a.path[(int64_t)b * a.path_stride + t];
        s_node[t] = node;
        if (node < t || node >= a.n_q) s_bad = 1;
    }
    __syncthreads();
    if (s_bad) {
        if (t == 0 && a.dev_status) a.dev_status[b] = 4;
        return;
    }
    // the moves (path positions whose node is not already in place), in path order
    if (a.path && t == 0) {
        int m = 0;
        for (int kk = 1; kk <= J; ++kk)
            if (s_node[kk] != kk) s_move[m++] = kk;
        s_moves = m;
    }
    __syncthreads();
    const int moves = s_moves;
    const int64_t seq = a.kv_off ? a.kv_off[b] : (int64_t)b * a.kv_sb;
    // item = ((move * Hkv + head) * 2 + tensor) * vpr + vector: move-major, so every round
    // covers whole moves before later ones
    const int per_move = a.Hkv * 2 * a.vpr;
    const int items = moves * per_move;
    constexpr int kRound = kCommitThreads * kVecPerThread;
    for (int r0 = 0; r0 < items; r0 += kRound) {
        u32x4 val[kVecPerThread];
        int64_t dst[kVecPerThread];  // byte offset of the destination, -1 for no item
        bool isv[kVecPerThread];
#pragma unroll
        for (int j = 0; j < kVecPerThread; ++j) {
            const int it = r0 + j * kCommitThreads + t;
            dst[j] = -1;
            isv[j] = false;
            if (it < items) {
                const int m = it / per_move, rem = it % per_move;
                const int g = rem / (2 * a.vpr), tensor = (rem / a.vpr) % 2, vec = rem % a.vpr;
                const int kk = s_move[m];
                const int64_t row = seq + (int64_t)g * a.kv_sh;
                const int64_t src = (row + (int64_t)(P + s_node[kk]) * a.kv_st) * a.esize + 16 * vec;
                dst[j] = (row + (int64_t)(P + kk) * a.kv_st) * a.esize + 16 * vec;
                isv[j] = tensor != 0;
                val[j] = *reinterpret_cast<const u32x4 *>((isv[j] ? a.v : a.k) + src);
            }
        }
        __syncthreads();  // every read of this round is done before any write
#pragma unroll
        for (int j = 0; j < kVecPerThread; ++j)
            if (dst[j] >= 0) *reinterpret_cast<u32x4 *>((isv[j] ? a.v : a.k) + dst[j]) = val[j];
        __syncthreads();  // this round's writes are done before the next round's reads
    }
    if (t == 0) {
        a.new_len[b] = P + 1 + J;
        if (a.dev_status) a.dev_status[b] = 0;
    }
}

}  // namespace

extern "C" sv_status sv_kv_commit(const sv_commit_desc *d, void *stream)
{
    if (!d) return SV_ERR_INVALID_ARG;
    if (d->dtype != SV_F32 && d->dtype != SV_BF16) return SV_ERR_INVALID_ARG;
    if (d->B < 0 || d->n_q < 1 || d->Hkv < 1 || d->D < 1) return SV_ERR_INVALID_ARG;
    if (!d->k || !d->v || !d->prefix_len || !d->accept_len || !d->new_len) return SV_ERR_INVALID_ARG;
    if (d->kv_sh < 0 || d->kv_st < 0 || (!d->kv_off && d->kv_sb < 0)) return SV_ERR_INVALID_ARG;
    if (d->path && (d->path_stride < 1 || d->path_stride > kMaxPath)) return SV_ERR_UNSUPPORTED;
    const int esize = d->dtype == SV_BF16 ? 2 : 4;
    const int64_t row_bytes = (int64_t)d->D * esize;
    // 16-byte vectors: rows, strides and base pointers aligned to 16 bytes
    const int64_t el16 = 16 / esize;
    if (row_bytes % 16 || d->kv_sh % el16 || d->kv_st % el16 || (!d->kv_off && d->kv_sb % el16) ||
        (((uintptr_t)d->k | (uintptr_t)d->v) & 15))
        return SV_ERR_UNSUPPORTED;
    if (d->B == 0) return SV_OK;
    CommitArgs a;
    a.k = (char *)d->k;
    a.v = (char *)d->v;
    a.kv_off = d->kv_off;
    a.kv_sb = d->kv_sb;
    a.kv_sh = d->kv_sh;
    a.kv_st = d->kv_st;
    a.esize = esize;
    a.B = d->B;
    a.n_q = d->n_q;
    a.Hkv = d->Hkv;
    a.vpr = (int)(row_bytes / 16);
    a.prefix_len = d->prefix_len;
    a.accept_len = d->accept_len;
    a.path = d->path;
    a.path_stride = d->path_stride;
    a.new_len = d->new_len;
    a.dev_status = d->dev_status;
    (void)hipGetLastError();
    hipLaunchKernelGGL(kv_commit_kernel, dim3(d->B), dim3(kCommitThreads), 0, (hipStream_t)stream, a);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}
