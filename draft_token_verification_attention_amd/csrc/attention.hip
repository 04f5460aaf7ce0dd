// attention.hip -- the multi-token attention of a verification pass.
//
// Sources: "Speculative decoding" (Zero to Frontier textbook, ch. 20, section 20.5):
// section "Checking several tokens costs about as much as writing one" (each new token
// attends to the whole cache and to the new tokens before it, a causal mask aligned to
// its bottom-right corner; the cost is reading the cache, which does not grow with k)
// and box "Token tree and tree attention" (node i sees the prefix, itself and its
// ancestors).  "Speculative-Decoding" (Medusa notes), section "Attention Tree".
//
// bf16 path (MFMA, gfx950 v_mfma_f32_32x32x16_bf16):
//   * The rows of one KV head are the n_q x G query rows that read it (grouped-query
//     packing, row n = i * G + g), so every K/V tile is read once for all of them.
//   * A block owns (sequence, KV head, row tile of 32*NWR rows, key split).  Its waves
//     form NWK key groups x NWR row waves: a key group stages 32-key tiles of K and V
//     through LDS (coalesced 16-byte loads, the next tile in registers while the current
//     one is computed), and each row wave of the group computes S^T = K Q^T and
//     O^T += V^T P^T for its 32 rows on MFMA.
//   * Online softmax in registers (log2 domain; the reference moves only when a row's
//     weights against it could grow past 2^16).  Key groups
//     merge through LDS; key splits are merged by attn_combine_kernel (log-sum-exp).
//   * Tiles the mask hides from every row of the block are never loaded (tree nodes of
//     other branches; chain positions after the block's last row).
//   * One row wave (decode): a plain (split, KV head, sequence) grid, K/V streamed with
//     nontemporal loads; with a dense cache and a grid of at most one block per CU, each
//     wave loads its first tile before the sequence length arrives.  Several row waves:
//     all blocks of one KV head are numbered onto one XCD (workgroup id mod 8), so the row
//     tiles that re-read its K/V share that XCD's L2.
// fp32 path: one wave per query row, lanes across the head dimension (VALU).
#include <hip/hip_ext.h>

#include "sv_common.h"

namespace {

using namespace sv;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// Native 16-byte vector: arrays of it stay in registers (arrays of the uint4 struct do not).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileKeys = 32;
constexpr int kMaxTiles = 1024;  // tiles per split (split_keys <= 32768)
constexpr int kMaxSplits = 64;   // key splits per sequence
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kPsumMax = 65536.0f;  // online softmax: largest weight against a stale reference

struct AttnArgs {
    const void *q;
    int64_t q_sb, q_st, q_sh;
    const void *k, *v;
    const int64_t *kv_off;  // or NULL: sequence b starts at element b * kv_sb
    int64_t kv_sh, kv_st, kv_sb;
    const int32_t *prefix_len;
    int max_prefix, tmax;   // tmax = max_prefix + n_q
    const uint32_t *tree_bits;
    int64_t tree_sb;
    int words, tree;
    void *out;
    int64_t o_sb, o_st, o_sh;
    float *lse;
    int B, n_q, Hq, Hkv, G, rows, RT, KG, nsplit, split_keys;
    float scale_log2;
    float *part;  // [KG*RT][nsplit][32*NWR][D] bf16: o / sum of each split
    float2 *pml;  // [KG*RT][nsplit][32*NWR]: (max in log2 units, sum) of each split
};

// 16-byte K/V load.  NT: with the nontemporal hint, for tiles that no other block re-reads
// (one-row-wave blocks): streamed K/V then does not evict from the L2 what other blocks
// still need (sequence lengths, queries, split partials).  Measured on the 64-sequence batch:
// 219 -> 202 us.
template <bool NT>
__device__ __forceinline__ u32x4 load_kv16(const char *p)
{
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    else return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u)
{
    return __builtin_bit_cast(bf16x8, u);
}

// s_waitcnt immediate that waits until at most n vector-memory loads are outstanding
// (vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their no-wait maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// ds_read_b64_tr_b16: within each group of 16 lanes, source lane r supplies the address of
// four consecutive 16-bit values M[r][0..3]; destination lane r receives
// (M[r / 4][r % 4], M[4 + r / 4][r % 4], M[8 + r / 4][r % 4], M[12 + r / 4][r % 4]).
__device__ __forceinline__ v4s lds_read_tr16(const char *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(p));
}

// Combine lane l with lane l ^ 32 (v_permlane32_swap: with both operands x, the two
// results hold x[l % 32] and x[l % 32 + 32] in every lane l).
__device__ __forceinline__ float half_swap_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Bit k of the result: key t0 + k is visible to the lane's row (query i).  Keys before P
// (the cached prefix) are visible to every row; keys at or past T are not; a new token
// j = t - P is visible when j <= i (chain) or when bit j of the row's tree mask is set (tree).
// Rows past the last (padding, never stored) see every key before T.  t0 < T.
__device__ __forceinline__ uint32_t tile_visibility(const AttnArgs &a, const uint32_t *bits_row, bool row_ok, int i,
                                                    int t0, int P, int T)
{
    const int nvalid = T - t0;
    const uint32_t valid = nvalid >= 32 ? 0xffffffffu : ((1u << nvalid) - 1u);
    if (!row_ok) return valid;
    const int j0 = t0 - P;  // new-token index of the tile's first key (negative: prefix keys)
    const uint32_t pre = j0 >= 0 ? 0u : (j0 <= -32 ? 0xffffffffu : ((1u << -j0) - 1u));
    uint32_t node;
    if (!a.tree) {
        // keys with j0 + k <= i
        const int last = i - j0;
        node = last < 0 ? 0u : (last >= 31 ? 0xffffffffu : ((2u << last) - 1u));
    } else if (j0 >= 0) {
        // bits j0 .. j0 + 31 of the row's mask (the words past its end read as 0)
        const int w = j0 >> 5, sh = j0 & 31;
        const uint32_t lo = bits_row[w];
        const uint32_t hi = (w + 1 < a.words) ? bits_row[w + 1] : 0u;
        node = sh ? ((lo >> sh) | (hi << (32 - sh))) : lo;
    } else {
        // bits 0 .. 31 + j0 of the row's mask, placed at k = -j0 ...
        node = j0 <= -32 ? 0u : (bits_row[0] << -j0);
    }
    return valid & (pre | node);
}

// ---------------------------------------------------------------------------
// SPEC (one-row-wave variant, kv_off NULL): each wave issues its first tile's loads before
// the sequence length is known.
template <int DH, int NWR, int NWK, bool SPEC>
__global__ __launch_bounds__(64 * NWR * NWK, 2) void attn_bf16_kernel(AttnArgs a)
{
    constexpr int ROWS_BLK = 32 * NWR;
    // LDS row pitches: K rows padded by 16 B (the 16-byte A-operand reads of 32 rows hit
    // distinct banks), V rows by 64 B (the transpose reads of 4 rows x 4 column groups per
    // 16 lanes hit distinct banks; with a 16 B pad they conflict 4-way)
    constexpr int KROW = DH * 2 + 16;
    constexpr int VROW = DH * 2 + 64;
    constexpr int TILE_BYTES = kTileKeys * KROW;
    constexpr int GROUP_BYTES = kTileKeys * (KROW + VROW);  // K then V
    constexpr int TILES_LDS = NWK * GROUP_BYTES;
    constexpr int NDB = DH / 32;                        // 32-wide d blocks of O^T
    constexpr int NKC = DH / 16;                        // 16-deep d chunks of S^T
    constexpr int COMB_LDS = NWR * NWK * 64 * (2 + (NWK > 1 ? NDB * 16 : 0)) * 4;
    constexpr int SMEM = TILES_LDS > COMB_LDS ? TILES_LDS : COMB_LDS;
    constexpr int LPR = DH / 8;                         // lanes per key row in a 16 B load
    constexpr int KPI = 64 / LPR;                       // key rows per wave load instruction
    constexpr int KPW = kTileKeys / NWR;                // key rows loaded per wave
    constexpr int NI = KPW / KPI;                       // load instructions per wave and tensor
    static_assert(NI >= 1 && KPW % KPI == 0, "tile split");
    static_assert(!SPEC || NWR == 1, "speculative first tile: one-row-wave variant");

    __shared__ __align__(16) char smem[SMEM];
    __shared__ uint16_t tile_list[kMaxTiles];
    __shared__ int s_count;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar tile math
    const int wk = wave % NWK;
    const int wr = wave / NWK;
    const int h = lane >> 5;          // half of the wave
    const int l32 = lane & 31;

    constexpr bool kDecode = (NWR == 1);
    // ---- block -> (kv group, row tile, split) ----
    // One row wave: a plain (split, KV head, sequence) grid.  Several row waves: all blocks
    // of a KV head are numbered onto one XCD (workgroup id mod 8), so the row tiles that
    // re-read its K/V share that XCD's L2.
    int kg, rt, s, b, kvh;
    if (kDecode) {
        s = blockIdx.x;
        kvh = blockIdx.y;
        b = blockIdx.z;
        kg = b * a.Hkv + kvh;
        rt = 0;
    } else {
        const int L = blockIdx.x;
        const int xcd = L & 7;
        const int slot = L >> 3;
        const int per_kg = a.RT * a.nsplit;
        kg = (slot / per_kg) * 8 + xcd;
        const int rem = slot % per_kg;
        rt = rem / a.nsplit;
        s = rem % a.nsplit;
        if (kg >= a.KG) return;
        b = kg / a.Hkv;
        kvh = kg % a.Hkv;
    }
    // this wave's 32 query rows (B operand of S^T = K Q^T): issued before anything waits
    const int rowbase = rt * ROWS_BLK;
    const int my_row = rowbase + wr * 32 + l32;
    const bool row_ok = my_row < a.rows;
    const int my_i = row_ok ? my_row / a.G : 0;
    bf16x8 qf[NKC];
    {
        const uint16_t *qrow = (const uint16_t *)a.q + (int64_t)b * a.q_sb + (int64_t)my_i * a.q_st +
                               (int64_t)(kvh * a.G + (row_ok ? my_row % a.G : 0)) * a.q_sh;
#pragma unroll
        for (int c = 0; c < NKC; ++c) {
            const uint4 u = *reinterpret_cast<const uint4 *>(qrow + 16 * c + 8 * h);
            qf[c] = as_bf16x8(u);
        }
    }
    const int SK = a.split_keys;
    const int64_t seq_off = SPEC ? (int64_t)b * a.kv_sb : (a.kv_off ? a.kv_off[b] : (int64_t)b * a.kv_sb);
    const uint16_t *kbase = (const uint16_t *)a.k + seq_off + (int64_t)kvh * a.kv_sh;
    const uint16_t *vbase = (const uint16_t *)a.v + seq_off + (int64_t)kvh * a.kv_sh;

    // ---- staging registers for this wave's share of a K/V tile ----
    u32x4 kreg[NI], vreg[NI];
    const int ld_key0 = wr * KPW + lane / LPR;
    const int ld_dc = lane % LPR;
    if constexpr (SPEC) {
        // The first tile of this wave (tile wk of the split), loaded while the sequence
        // length is still in flight.  Every sequence's slot holds tmax tokens, so rows are
        // clamped below tmax; rows at or past the sequence's end are zeroed before use.
        const int t0 = s * SK + wk * kTileKeys;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int64_t o = (int64_t)min(t0 + ld_key0 + j * KPI, a.tmax - 1) * a.kv_st + 8 * ld_dc;
            kreg[j] = load_kv16<true>(reinterpret_cast<const char *>(kbase + o));
            vreg[j] = load_kv16<true>(reinterpret_cast<const char *>(vbase + o));
        }
    }
    const int P = a.prefix_len[b];
    const int T = P + a.n_q;
    // a sequence whose prefix is negative or longer than max_prefix reads nothing and
    // reports NaN rows
    const bool overflow = P > a.max_prefix || P < 0;
    const int ns = overflow ? a.nsplit : (T + SK - 1) / SK;
    if (s >= ns) return;
    const int kstart = s * SK;
    const int kend = overflow ? kstart : min(kstart + SK, T);
    const int row_hi = min(rowbase + ROWS_BLK, a.rows) - 1;
    const int i_lo = rowbase / a.G, i_hi = row_hi / a.G;

    const uint32_t *bits_b = a.tree ? a.tree_bits + (int64_t)b * a.tree_sb : nullptr;

    // ---- the tiles some row of this block can see ----
    // One row wave (few rows): every tile from the split start up to the block's last
    // visible key, in order (small trees keep all their node tiles; the mask hides keys).
    // Several row waves: an explicit list (wave 0, ballot compaction), which skips the
    // node tiles that no row of the block can see.
    int count;
    if (kDecode) {
        const int vis_end = a.tree ? kend : min(kend, P + i_hi + 1);
        count = vis_end > kstart ? (vis_end - kstart + kTileKeys - 1) / kTileKeys : 0;
    }
    if (!kDecode && wave == 0) {
        const int ntile = (kend - kstart + kTileKeys - 1) / kTileKeys;
        // Tree: the OR of the block's node rows over the mask words that cover the split's
        // new tokens, into LDS (the tile buffers, not in use yet).  Lanes take words; each
        // lane's rows go in batches of independent loads.
        uint32_t *or_w = reinterpret_cast<uint32_t *>(smem);
        const int jbeg = max(kstart - P, 0);  // the split's first new token
        const int jend = min(kend, T) - P;    // one past its last (<= jbeg: none)
        const int w0 = jbeg >> 5;
        const int nw = jend > jbeg ? ((jend - 1) >> 5) - w0 + 1 : 0;
        if (a.tree) {
            for (int wl = lane; wl < nw; wl += 64) {
                const uint32_t *col = bits_b + w0 + wl;
                uint32_t acc = 0u;
                int i = i_lo;
                for (; i + 8 <= i_hi + 1; i += 8) {
                    uint32_t v[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) v[u] = col[(int64_t)(i + u) * a.words];
#pragma unroll
                    for (int u = 0; u < 8; ++u) acc |= v[u];
                }
                for (; i <= i_hi; ++i) acc |= col[(int64_t)i * a.words];
                or_w[wl] = acc;
            }
            __builtin_amdgcn_wave_barrier();
        }
        int count = 0;
        for (int t0i = 0; t0i < ntile; t0i += 64) {
            const int tt = t0i + lane;
            bool inc = false;
            if (tt < ntile) {
                const int t0 = kstart + tt * kTileKeys;
                if (t0 < P) {
                    inc = true;
                } else {
                    const int j0 = t0 - P;
                    if (!a.tree) {
                        inc = j0 <= i_hi;
                    } else {
                        // new tokens j0 .. jl, all inside the words or_w holds
                        const int jl = min(j0 + kTileKeys, a.n_q) - 1;
                        for (int w = j0 >> 5; w <= (jl >> 5); ++w) {
                            const uint32_t word = or_w[w - w0];
                            const int lo = max(j0 - 32 * w, 0), hi = min(jl - 32 * w, 31);
                            const uint32_t m_hi = hi == 31 ? 0xffffffffu : ((1u << (hi + 1)) - 1u);
                            const uint32_t m_lo = ~((1u << lo) - 1u);
                            if (word & m_hi & m_lo) inc = true;
                        }
                    }
                }
            }
            const uint64_t mask = __ballot(inc);
            const int pos = count + __popcll(mask & ((1ull << lane) - 1ull));
            if (inc) tile_list[pos] = (uint16_t)tt;
            count += __popcll(mask);
        }
        if (lane == 0) s_count = count;
    }
    if (!kDecode) {
        __syncthreads();
        count = s_count;
    }
    const int niter = (count + NWK - 1) / NWK;
    auto tile_start = [&](int li) {
        return kstart + (kDecode ? li : __builtin_amdgcn_readfirstlane((int)tile_list[li])) * kTileKeys;
    };

    const uint32_t *my_bits = a.tree ? bits_b + (int64_t)my_i * a.words : nullptr;

    // Tile loads address a uniform tile base (scalar registers) plus per-lane byte offsets
    // that are the same for every full tile.  In the last, partial tile, key rows past the
    // end of the cache re-read the last valid row (in bounds); the mask hides those keys,
    // so their finite values add 0.
    uint32_t voff[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) voff[j] = 2u * ((uint32_t)(ld_key0 + j * KPI) * (uint32_t)a.kv_st + 8u * ld_dc);
    int t0_cur = 0;  // several row waves: start of the tile loaded last (read from the list once)
    auto issue_loads = [&](int it) {
        const int li = it * NWK + wk;
        if (li < count) {
            const int t0 = tile_start(li);
            if constexpr (!kDecode) t0_cur = t0;
            const char *kb = reinterpret_cast<const char *>(kbase + (int64_t)t0 * a.kv_st);
            const char *vb = reinterpret_cast<const char *>(vbase + (int64_t)t0 * a.kv_st);
            const int lim = T - 1 - t0;  // >= 0: every tile starts inside the cache
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const uint32_t o = (t0 + kTileKeys <= T)
                                       ? voff[j]
                                       : 2u * ((uint32_t)min(ld_key0 + j * KPI, lim) * (uint32_t)a.kv_st + 8u * ld_dc);
                kreg[j] = load_kv16<kDecode>(kb + o);
                vreg[j] = load_kv16<kDecode>(vb + o);
            }
        }
    };

    char *gK = smem + wk * GROUP_BYTES;
    char *gV = gK + TILE_BYTES;

    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[db][v] = 0.0f;
    float m_run = -INFINITY;
    float l_run = 0.0f;

    // One row wave: each wave streams its own tiles through its own LDS buffers, so the
    // loop needs no block barrier (a wave's LDS accesses complete in issue order).
    // Several row waves share a tile: barriers around the LDS writes.
    // Q must have landed before the first MFMA.  Left to the compiler, that wait merges into
    // the first MFMA of every tile as a wait for all outstanding loads, which defeats the
    // prefetch; so the wait is explicit, here.  One row wave: the first tile's loads go out
    // first, and the wait covers Q alone (issued before them), leaving the tile in flight
    // (1-2% on the 64-sequence batch).  Every wave issues that tile without a branch (a
    // branch there makes the compiler copy registers that are still loading): a wave past
    // the split's last tile re-reads that tile, a block with no tile reads its own first Q
    // row.  Q itself is loaded by every lane (padding rows read the block's first row; their
    // results are never stored), again without a branch.
    if constexpr (kDecode && !SPEC) {
        const bool any = count > 0;
        const int t0 = kstart + (any ? min(wk, count - 1) : 0) * kTileKeys;
        const char *qsafe = reinterpret_cast<const char *>((const uint16_t *)a.q + (int64_t)b * a.q_sb +
                                                           (int64_t)(kvh * a.G) * a.q_sh);
        const char *kb = any ? reinterpret_cast<const char *>(kbase + (int64_t)t0 * a.kv_st) : qsafe;
        const char *vb = any ? reinterpret_cast<const char *>(vbase + (int64_t)t0 * a.kv_st) : qsafe;
        const int lim = T - 1 - t0;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const uint32_t o = !any ? 0u
                               : (t0 + kTileKeys <= T)
                                   ? voff[j]
                                   : 2u * ((uint32_t)min(ld_key0 + j * KPI, lim) * (uint32_t)a.kv_st + 8u * ld_dc);
            kreg[j] = load_kv16<true>(kb + o);
            vreg[j] = load_kv16<true>(vb + o);
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NI));
    } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(SPEC ? 2 * NI : 0));
        if (!SPEC && niter > 0) issue_loads(0);
    }
    // Q is complete here: hand it on as a fresh value, so that no wait for it (which would
    // also wait for the tile in flight) lands in the loop
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
        u32x4 t = __builtin_bit_cast(u32x4, qf[c]);
        asm volatile("" : "+v"(t));
        qf[c] = __builtin_bit_cast(bf16x8, t);
    }
    const int my_iters = kDecode ? (count - wk + NWK - 1) / NWK : niter;
    // rows of the speculative first tile at or past the end of the sequence (zeroed)
    const int spec_lim = T - (kstart + wk * kTileKeys);
    for (int it = 0; it < my_iters; ++it) {
        const int li = it * NWK + wk;
        const bool have = li < count;
        if (!kDecode) __syncthreads();  // the previous tile is no longer read
        if (have) {
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int key = ld_key0 + j * KPI;
                u32x4 kv = kreg[j], vv = vreg[j];
                if (SPEC && it == 0 && key >= spec_lim) {
                    kv = u32x4{0u, 0u, 0u, 0u};
                    vv = u32x4{0u, 0u, 0u, 0u};
                }
                *reinterpret_cast<u32x4 *>(gK + key * KROW + 16 * ld_dc) = kv;
                *reinterpret_cast<u32x4 *>(gV + key * VROW + 16 * ld_dc) = vv;
            }
        }
        if (!kDecode) __syncthreads();
        const int t0 = kDecode ? tile_start(li) : t0_cur;
        if (it + 1 < my_iters) issue_loads(it + 1);
        if (!have) continue;

        // S^T (32 keys x 32 rows) = K (keys x d) . Q^T (d x rows), masked, into sv.  It reads
        // K from LDS only, so it can run again while the tile is there.
        auto scores = [&](float (&sv)[16]) {
            // One row wave: two independent MFMA chains over the even and odd d chunks (half
            // the dependent-MFMA latency on a latency-bound path); several: one chain (other
            // waves hide its latency, and the 16 adds that join two chains are VALU time the
            // MFMA-bound path lacks)
            constexpr bool kTwoChains = kDecode;
            f32x16 sacc, sacc1;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                sacc[v] = 0.0f;
                sacc1[v] = 0.0f;
            }
#pragma unroll
            for (int c = 0; c < NKC; c += 2) {
                const bf16x8 kf0 = *reinterpret_cast<const bf16x8 *>(gK + l32 * KROW + (16 * c + 8 * h) * 2);
                const bf16x8 kf1 = *reinterpret_cast<const bf16x8 *>(gK + l32 * KROW + (16 * c + 16 + 8 * h) * 2);
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf0, qf[c], sacc, 0, 0, 0);
                if constexpr (kTwoChains)
                    sacc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf1, qf[c + 1], sacc1, 0, 0, 0);
                else
                    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf1, qf[c + 1], sacc, 0, 0, 0);
            }
            if constexpr (kTwoChains) {
#pragma unroll
                for (int v = 0; v < 16; ++v) sacc[v] += sacc1[v];
            }
            // lane (row l32, half h) holds keys 8*(v/4) + 4*h + v%4 of the tile
            if (t0 + kTileKeys > P) {
                // the tile reaches the new tokens (or the end of the cache): one visibility word
                // for the lane's row, then a select per score
                // (shifted by the lane's half first, so each score's bit sits at a constant)
                const uint32_t vis = tile_visibility(a, my_bits, row_ok, my_i, t0, P, T) >> (4 * h);
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    sv[v] = (vis & (1u << (8 * (v >> 2) + (v & 3)))) ? sacc[v] : -INFINITY;
            } else {
#pragma unroll
                for (int v = 0; v < 16; ++v) sv[v] = sacc[v];
            }
        };
        float sv[16];
        scores(sv);
        // Online softmax against a reference m_run (log2 units) that moves only when it must.
        // Weights are taken against the current reference first; while every lane's 16 weights
        // sum to at most kPsumMax (a finite sum: the reference is set and no weight overflowed),
        // they stand, and the tile costs no row max and no rescale.  Otherwise (a row's first
        // visible keys, or scores far above the reference) the row max of the tile is taken
        // on the raw scores (scale > 0), the reference moves to it, the weights are taken again
        // and the accumulators rescaled.  Every weight stands at most kPsumMax, and the result
        // does not depend on where the reference sits (exact in the final l and O).
        float p[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) p[v] = exp2_fast(fmaf(sv[v], a.scale_log2, -m_run));
        float psum = p[0];
#pragma unroll
        for (int v = 1; v < 16; ++v) psum += p[v];
        if (__ballot(!(psum <= kPsumMax))) {
            // the scores again, from LDS (the memory clobber keeps the compiler from holding
            // the first pass's K fragments live through the weights instead)
            asm volatile("" ::: "memory");
            scores(sv);
            float mloc = sv[0];
#pragma unroll
            for (int v = 1; v < 16; ++v) mloc = fmaxf(mloc, sv[v]);
            mloc = half_swap_max(mloc);  // the row's other 16 keys sit in lane l ^ 32
            const float m_new = fmaxf(m_run, mloc * a.scale_log2);
            // a row with no visible key yet (m_new = -inf) subtracts 0 instead, so its weights
            // are exp2(-inf) = 0 and its alpha 0 (l and O are still zero there)
            const float m_sub = (m_new == -INFINITY) ? 0.0f : m_new;
            const float alpha = exp2_fast(m_run - m_sub);  // m_run == -inf gives 0
#pragma unroll
            for (int v = 0; v < 16; ++v) p[v] = exp2_fast(fmaf(sv[v], a.scale_log2, -m_sub));
            psum = 0.0f;
#pragma unroll
            for (int v = 0; v < 16; ++v) psum += p[v];
            l_run *= alpha;
            m_run = m_new;
            // rescale the accumulators only when some row's reference moved (never needed on
            // a wave's first tile, where they are still zero)
            if (it > 0 && __ballot(alpha != 1.0f)) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;
            }
        }
        l_run += psum;

        // P^T as the B operand: k index 8*h + j <-> key 16*c + 8*(j/4) + 4*h + j%4
        bf16x8 pb[2];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int j = 0; j < 8; ++j) pb[c][j] = (__bf16)p[8 * c + j];

        // O^T (d x rows) += V^T (d x keys) . P^T (keys x rows).  Lane (d, h) needs V at
        // column d for keys 16c + 4h + 0..3 and 16c + 8 + 4h + 0..3: two LDS transpose reads
        // (within each 16-lane group, source lane r addresses key row r / 4 of the group's
        // four and the four columns starting at 4 (r % 4); destination lane r gets column
        // r of those four rows).
        const int g16 = lane >> 4, r16 = lane & 15;
        const char *vsrc = gV + (4 * (g16 >> 1) + (r16 >> 2)) * VROW + 2 * (16 * (g16 & 1) + 4 * (r16 & 3));
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const char *p0 = vsrc + 16 * c * VROW + 64 * db;
                const v4s lo = lds_read_tr16(p0), hi = lds_read_tr16(p0 + 8 * VROW);
                const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[c], oacc[db], 0, 0, 0);
            }
        }
    }

    // ---- merge the NWK key groups of each row wave (through LDS) ----
    // Every wave rescales its accumulators to the common row max, writes them to LDS, and
    // then sums (in fixed wave order: deterministic) and stores one NWK-th of the row
    // wave's output elements.  Element e = db*16 + v of lane (row l32, half h) is
    // d = 32*db + 8*(v/4) + 4*h + v%4.
    constexpr int NE = NDB * 16;                 // accumulator elements per lane
    constexpr int EPW = NE / NWK;                // elements each key wave stores
    static_assert(NE % NWK == 0 && EPW % 4 == 0, "merge split");
    float *mls = reinterpret_cast<float *>(smem);                       // [NWR][NWK][2][64]
    float *accs = mls + NWR * NWK * 2 * 64;                             // [NWR][NWK][NE][64]
    float row_inv_l, row_m;
    float mrg[EPW];                              // this wave's merged share (NWK > 1)
    {
        // the merge scratch overlays the tile buffers: wait until no wave reads a tile
        if (NWK > 1 || NWR > 1) __syncthreads();
        float *my_ml = mls + ((wr * NWK + wk) * 2) * 64;
        my_ml[lane] = m_run;
        my_ml[64 + lane] = l_run;
        if (NWK > 1) __syncthreads();
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < NWK; ++k) M = fmaxf(M, mls[((wr * NWK + k) * 2) * 64 + lane]);
        float Lr = 0.0f;
#pragma unroll
        for (int k = 0; k < NWK; ++k) {
            const float mk = mls[((wr * NWK + k) * 2) * 64 + lane];
            const float lk = mls[((wr * NWK + k) * 2) * 64 + 64 + lane];
            Lr += (mk == -INFINITY) ? 0.0f : lk * exp2_fast(mk - M);
        }
        Lr = half_swap_sum(Lr);  // the other half of the row's keys
        row_m = M;
        row_inv_l = Lr;
        if (NWK > 1) {
            const float f = (m_run == -INFINITY) ? 0.0f : exp2_fast(m_run - M);
            float *my_acc = accs + ((wr * NWK + wk) * NE) * 64;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) my_acc[(db * 16 + v) * 64 + lane] = oacc[db][v] * f;
            __syncthreads();
            // this wave's share: elements [wk*EPW, (wk+1)*EPW), summed over the key waves
#pragma unroll
            for (int e = 0; e < EPW; ++e) {
                float sum = 0.0f;
#pragma unroll
                for (int k = 0; k < NWK; ++k) sum += accs[((wr * NWK + k) * NE + wk * EPW + e) * 64 + lane];
                mrg[e] = sum;  // element wk*EPW + e
            }
        }
    }
    const int e0 = (NWK > 1) ? wk * EPW : 0;      // first element this wave stores
    const int ne = (NWK > 1) ? EPW : NE;           // elements this wave stores
    auto elem = [&](int j) -> float {              // j-th element this wave stores
        return (NWK > 1) ? mrg[j] : oacc[j / 16][j % 16];
    };
    const float l_row = row_inv_l;
    if (!row_ok) return;
    const int hq = kvh * a.G + my_row % a.G;

    if (a.nsplit == 1) {
        // one split: normalize and store straight from registers
        const float inv = overflow ? __int_as_float(0x7fc00000) : 1.0f / l_row;
        uint16_t *o = (uint16_t *)a.out + (int64_t)b * a.o_sb + (int64_t)my_i * a.o_st + (int64_t)hq * a.o_sh;
#pragma unroll
        for (int j = 0; j < ne; j += 4) {
            const int e = e0 + j;
            const int d = 32 * (e / 16) + 8 * ((e % 16) / 4) + 4 * h;
            uint2 pk;
            pk.x = (uint32_t)f32_to_bf16(elem(j) * inv) | ((uint32_t)f32_to_bf16(elem(j + 1) * inv) << 16);
            pk.y = (uint32_t)f32_to_bf16(elem(j + 2) * inv) | ((uint32_t)f32_to_bf16(elem(j + 3) * inv) << 16);
            *reinterpret_cast<uint2 *>(o + d) = pk;
        }
        if (a.lse && h == 0 && wk == 0)
            a.lse[((int64_t)b * a.n_q + my_i) * a.Hq + hq] =
                overflow ? __int_as_float(0x7fc00000) : (row_m + log2f(l_row)) * kLn2;
        return;
    }

    // several splits: store this split's partial -- o / sum in bf16, (max in log2 units, sum)
    // in fp32 -- for the combine kernel, which runs after this kernel completes.  These
    // writes reach HBM while other blocks are still streaming K/V, and there they cost far
    // more than their size (a plain streaming read with fp32 partials' worth of writes added
    // slows from 6.7 to 5.6 TB/s; writes that stay in L2 cost nothing), so the partial o is
    // stored normalized and in bf16: half the bytes, 197.6 -> 186.6 us on the 64-sequence
    // batch.  o / sum is a convex combination of V rows, so its rounding error is at most
    // 2^-9 of the largest |V| element it averages, and the combined output (again a convex
    // combination) carries at most that on top of its own bf16 rounding.
    const int gidx = kg * a.RT + rt;
    const int64_t prow = ((int64_t)gidx * a.nsplit + s) * ROWS_BLK + wr * 32 + l32;
    uint16_t *pr = reinterpret_cast<uint16_t *>(a.part) + prow * DH;
    const float pinv = l_row > 0.0f ? 1.0f / l_row : 0.0f;
#pragma unroll
    for (int j = 0; j < ne; j += 4) {
        const int e = e0 + j;
        const int d = 32 * (e / 16) + 8 * ((e % 16) / 4) + 4 * h;
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(elem(j) * pinv) | ((uint32_t)f32_to_bf16(elem(j + 1) * pinv) << 16);
        pk.y = (uint32_t)f32_to_bf16(elem(j + 2) * pinv) | ((uint32_t)f32_to_bf16(elem(j + 3) * pinv) << 16);
        *reinterpret_cast<uint2 *>(pr + d) = pk;
    }
    if (h == 0 && wk == 0) a.pml[prow] = make_float2(row_m, l_row);
}

// ---------------------------------------------------------------------------
// Split combine.  Per row: M = max_s m_s, L = sum_s l_s 2^(m_s - M),
// O = sum_s o_s 2^(m_s - M) / L.  A row is served by NSL split lanes x column lanes, each
// column lane owning kCombVec float4 of the row (1 for small grids, latency first; 4 for
// large ones, fewer blocks); split lane sl reads splits sl, sl + NSL, ...,
// SPT of them at most, all loads issued at once (clamped in-bounds, weighted 0 past the
// row's last split).  The split lanes are summed through LDS in fixed order.
// Tasks (row chunk, kv group x row tile); a grid smaller than the task count loops.
// ---------------------------------------------------------------------------
constexpr int kCombThreads = 256;

template <int DH, int ROWS_BLK, int NSL, int SPT, int kCombVec>
__global__ __launch_bounds__(kCombThreads) void attn_combine_kernel(AttnArgs a, int nrc, int ntask)
{
    constexpr int L4 = DH / 4 / kCombVec;         // column lanes per row
    constexpr int RL = NSL * L4;                  // threads per row
    constexpr int CR = kCombThreads / RL;         // rows per block
    static_assert(CR >= 1 && kCombThreads % RL == 0, "combine layout");
    __shared__ float s_m[kCombThreads];
    __shared__ float4 s_o[kCombVec][kCombThreads];
    __shared__ float s_l[kCombThreads];
    const int rl = threadIdx.x / RL;              // row within the block
    const int sl = (threadIdx.x / L4) % NSL;      // split lane
    const int cl = threadIdx.x % L4;              // column lane: float4 columns cl + L4 * v
    for (int t = blockIdx.x; t < ntask; t += gridDim.x) {
        if (t != (int)blockIdx.x) __syncthreads();  // the previous task's LDS reads are done
        const int gidx = t / nrc;
        const int kg = gidx / a.RT, rt = gidx % a.RT;
        const int b = kg / a.Hkv, kvh = kg % a.Hkv;
        const int P = a.prefix_len[b];
        const int T = P + a.n_q;
        const bool overflow = P > a.max_prefix || P < 0;
        const int ns = overflow ? a.nsplit : (T + a.split_keys - 1) / a.split_keys;
        const int r = (t % nrc) * CR + rl;        // row within the tile
        const int row = rt * ROWS_BLK + r;
        const bool ok = r < ROWS_BLK && row < a.rows;
        const int rr = ok ? r : 0;                // in-bounds row for the (unused) loads of idle rows
        const int64_t pg = (int64_t)gidx * a.nsplit * ROWS_BLK;
        auto row_of = [&](int u) { return pg + (int64_t)u * ROWS_BLK + rr; };  // partial row of split u
        const int nmine = ns > sl ? (ns - sl + NSL - 1) / NSL : 0;  // splits this lane owns

        float4 o[SPT][kCombVec];
        float2 ml[SPT];
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
            const int64_t pr = row_of(min(sl + k * NSL, ns - 1));
            const uint16_t *rp = reinterpret_cast<const uint16_t *>(a.part) + pr * DH;
#pragma unroll
            for (int v = 0; v < kCombVec; ++v) {
                const uint2 u = *reinterpret_cast<const uint2 *>(rp + 4 * (cl + L4 * v));
                o[k][v] = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                                      __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
            }
            ml[k] = a.pml[pr];
        }
        float mloc = -INFINITY;
#pragma unroll
        for (int k = 0; k < SPT; ++k)
            if (k < nmine) mloc = fmaxf(mloc, ml[k].x);
        s_m[threadIdx.x] = mloc;
        __syncthreads();
        float M = -INFINITY;
#pragma unroll
        for (int q = 0; q < NSL; ++q) M = fmaxf(M, s_m[rl * RL + q * L4 + cl]);
        float4 acc[kCombVec];
#pragma unroll
        for (int v = 0; v < kCombVec; ++v) acc[v] = make_float4(0.f, 0.f, 0.f, 0.f);
        float lsum = 0.0f;
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
            const float w = (k < nmine && ml[k].x != -INFINITY) ? ml[k].y * exp2_fast(ml[k].x - M) : 0.0f;
#pragma unroll
            for (int v = 0; v < kCombVec; ++v) {
                acc[v].x += o[k][v].x * w;
                acc[v].y += o[k][v].y * w;
                acc[v].z += o[k][v].z * w;
                acc[v].w += o[k][v].w * w;
            }
            lsum += w;
        }
        if (NSL > 1) {
#pragma unroll
            for (int v = 0; v < kCombVec; ++v) s_o[v][threadIdx.x] = acc[v];
            s_l[threadIdx.x] = lsum;
            __syncthreads();
            lsum = 0.0f;
#pragma unroll
            for (int v = 0; v < kCombVec; ++v) acc[v] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int q = 0; q < NSL; ++q) {  // fixed order: deterministic
                const int src = rl * RL + q * L4 + cl;
#pragma unroll
                for (int v = 0; v < kCombVec; ++v) {
                    const float4 tq = s_o[v][src];
                    acc[v].x += tq.x;
                    acc[v].y += tq.y;
                    acc[v].z += tq.z;
                    acc[v].w += tq.w;
                }
                lsum += s_l[src];
            }
        }
        if (ok && sl == 0) {
            const float L = lsum;
            const float inv = overflow ? __int_as_float(0x7fc00000) : 1.0f / L;
            const int i = row / a.G;
            const int hq = kvh * a.G + row % a.G;
            uint16_t *out = (uint16_t *)a.out + (int64_t)b * a.o_sb + (int64_t)i * a.o_st + (int64_t)hq * a.o_sh;
#pragma unroll
            for (int v = 0; v < kCombVec; ++v) {
                uint2 pk;
                pk.x = (uint32_t)f32_to_bf16(acc[v].x * inv) | ((uint32_t)f32_to_bf16(acc[v].y * inv) << 16);
                pk.y = (uint32_t)f32_to_bf16(acc[v].z * inv) | ((uint32_t)f32_to_bf16(acc[v].w * inv) << 16);
                *reinterpret_cast<uint2 *>(out + 4 * (cl + L4 * v)) = pk;
            }
            if (a.lse && cl == 0)
                a.lse[((int64_t)b * a.n_q + i) * a.Hq + hq] =
                    overflow ? __int_as_float(0x7fc00000) : (M + log2f(L)) * kLn2;
        }
    }
}

// ---------------------------------------------------------------------------
// fp32: one wave per (sequence, row, query head); lane owns d = lane (+64)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a, int D)
{
    const int r = blockIdx.x;
    const int h = r % a.Hq;
    const int i = (r / a.Hq) % a.n_q;
    const int b = r / (a.Hq * a.n_q);
    const int lane = threadIdx.x;
    const int kvh = h / a.G;
    const int P = a.prefix_len[b];
    const bool overflow = P > a.max_prefix || P < 0;  // reads nothing, reports NaN
    const int T = overflow ? 0 : P + a.n_q;
    const float *q = (const float *)a.q + (int64_t)b * a.q_sb + (int64_t)i * a.q_st + (int64_t)h * a.q_sh;
    const int64_t seq_off = a.kv_off ? a.kv_off[b] : (int64_t)b * a.kv_sb;
    const float *kb = (const float *)a.k + seq_off + (int64_t)kvh * a.kv_sh;
    const float *vb = (const float *)a.v + seq_off + (int64_t)kvh * a.kv_sh;
    const uint32_t *bits = a.tree ? a.tree_bits + (int64_t)b * a.tree_sb + (int64_t)i * a.words : nullptr;
    const bool two = D > 64;
    const float q0 = q[lane];
    const float q1 = two ? q[lane + 64] : 0.0f;
    float m = -INFINITY, l = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int t = 0; t < T; ++t) {
        if (t >= P) {
            const int j = t - P;
            const bool vis = a.tree ? ((bits[j >> 5] >> (j & 31)) & 1u) : (j <= i);
            if (!vis) continue;
        }
        const float *kr = kb + (int64_t)t * a.kv_st;
        float part = q0 * kr[lane];
        if (two) part += q1 * kr[lane + 64];
        const float sc = wave_sum(part) * a.scale_log2;
        const float mn = fmaxf(m, sc);
        const float f = exp2_fast(m - mn);
        const float pw = exp2_fast(sc - mn);
        const float *vr = vb + (int64_t)t * a.kv_st;
        l = l * f + pw;
        o0 = o0 * f + pw * vr[lane];
        if (two) o1 = o1 * f + pw * vr[lane + 64];
        m = mn;
    }
    float *o = (float *)a.out + (int64_t)b * a.o_sb + (int64_t)i * a.o_st + (int64_t)h * a.o_sh;
    const float qnan = __int_as_float(0x7fc00000);
    o[lane] = overflow ? qnan : o0 / l;
    if (two) o[lane + 64] = overflow ? qnan : o1 / l;
    if (a.lse && lane == 0)
        a.lse[((int64_t)b * a.n_q + i) * a.Hq + h] = overflow ? qnan : (m + log2f(l)) * kLn2;
}

// ---------------------------------------------------------------------------
// launch planning (host)
// ---------------------------------------------------------------------------
struct Plan {
    int variant;  // 0: fp32, 1: (NWR=1, NWK=4), 2: (NWR=2, NWK=2), 3: (NWR=4, NWK=1)
    int NWR, NWK, rows, RT, KG, nsplit, split_keys, kg_pad;
    size_t part_bytes, o_bytes, cnt_bytes, total;  // part_bytes = o partials + (max, sum) pairs
    unsigned blocks;
    int max_blocks;  // resident-block budget of the looping combine (set at launch)
    bool spec;       // speculative first tile (set at launch)
    int gsplit;      // split extent of the one-row-wave grid (odd when nsplit > 1)
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static bool plan_attention(const sv_attn_desc *d, int cu_count, Plan &p)
{
    p = Plan{};
    if (d->dtype == SV_F32) {
        p.variant = 0;
        p.total = 0;
        return true;
    }
    const int G = d->Hq / d->Hkv;
    p.rows = d->n_q * G;
    // 64-row blocks (two key waves each: half the tiles per wave, twice the row tiles) beat
    // 128-row ones while the cache is short, and for a few hundred rows when they pad fewer
    // rows.  Measured, random trees with 4 query heads per KV head (128-row -> 64-row us):
    //   2048-key cache: 516 rows 37.3 -> 28.0, 1028 rows 51.4 -> 46.3, 4100 rows 153.5 -> 114.3;
    //   4096: 516 rows 47.4 -> 39.2, 1028 rows 66.7 -> 68.7, 4100 rows 223.0 -> 202.0;
    //   8192: 1028 rows 98.8 -> 115.6, 4100 rows 356.0 -> 372.8;
    //   16384: 260 rows 74.4 -> 70.0, 516 rows 106.1 -> 110.2, 4100 rows 658.9 -> 703.6.
    const int pad64 = (p.rows + 63) / 64 * 64 - p.rows, pad128 = (p.rows + 127) / 128 * 128 - p.rows;
    const bool short_cache = (int64_t)d->max_prefix + d->n_q <= 6144;
    if (p.rows <= 32) {
        p.variant = 1; p.NWR = 1; p.NWK = 4;
    } else if (p.rows <= 64 || (p.rows <= 8192 && short_cache) || (p.rows <= 320 && pad64 < pad128)) {
        p.variant = 2; p.NWR = 2; p.NWK = 2;
    } else {
        p.variant = 3; p.NWR = 4; p.NWK = 1;
    }
    const int rows_blk = 32 * p.NWR;
    p.RT = (p.rows + rows_blk - 1) / rows_blk;
    p.KG = d->B * d->Hkv;
    p.kg_pad = (p.KG + 7) / 8 * 8;
    const int64_t Tmax = (int64_t)d->max_prefix + d->n_q;
    const int64_t groups = (int64_t)p.KG * p.RT > 0 ? (int64_t)p.KG * p.RT : 1;
    const int64_t unit = kTileKeys;
    int64_t sk;
    if (d->split_keys > 0) {
        sk = ((int64_t)d->split_keys + unit - 1) / unit * unit;
    } else if (p.variant == 1) {
        // Few query rows: splitting keys is cheap (a partial is at most 32 rows).  Aim at
        // about 2048 splits in all, which balances uneven sequence lengths over the 256 CUs
        // (two 4-wave blocks per CU), keeping splits between 256 keys (shorter ones cost
        // more in partials and launch than they gain) and 4096.
        // Splits are a power of two long (measured: 1024-key splits stream a 64-sequence
        // batch a third faster than 1056-key ones).  On that batch (8197-key bound):
        // 2048-key splits 198.6 + 12.9 us (main + combine), 1024-key 200.0 + 14.6, 4096-key
        // 224.6 + 9.3, 512-key 212.4 + 18.3.
        const int64_t want = (Tmax * groups + 2047) / 2048;
        sk = 256;
        while (sk * 2 <= want && sk < 4096) sk *= 2;
        // Batches: splits of at least 1024 keys once the cache passes 2048 keys (8 or more
        // sequences of 8 KV heads) or 4096 keys (4 or more), and no split at all for short
        // caches with 8 or more sequences, which also saves the combine.  Measured, 6 query
        // rows x 32 query heads / 8 KV heads, us before -> after:
        //   B=8: 2048 keys 25.1 -> 22.4, 8192 66.2 -> 56.2;  B=4: 16384 keys 63.7 -> 53.6;
        //   B=16: 1024 keys 26.1 -> 19.5, 4096 67.8 -> 58.9;  B=64: 512 keys 43.5 -> 27.1,
        //   1024 keys 72.7 -> 47.8.  (B=2 and B=4 on 2048 keys lose with 1024-key splits.)
        if ((groups >= 64 && Tmax > 2048) || (groups >= 32 && Tmax >= 4096)) sk = sk < 1024 ? 1024 : sk;
        if (groups >= 64 && Tmax <= 2048) sk = (Tmax + unit - 1) / unit * unit;
        // A grid that 256-key splits leave within the CUs (one sequence, a few): shorter
        // splits, up to about three quarters of the CUs in blocks, at least 128 keys.  The 8B
        // chain (8 KV heads, 4102 keys): 256-key splits 10.1 us, 224 9.8, 192 9.5, 160 9.6,
        // 128 10.4 (more blocks than CUs).
        if (groups * ((Tmax + 255) / 256) <= cu_count) {
            const int64_t want = 3 * (int64_t)cu_count / 4;
            int64_t s2 = (Tmax * groups + want - 1) / want;
            s2 = (s2 + unit - 1) / unit * unit;
            if (s2 < 128) s2 = 128;
            if (s2 < sk) sk = s2;
        }
    } else {
        // Many rows per block: a partial (32 NWR rows x D, and a (max, sum) pair per row,
        // written and read back) costs about as much as the K/V of 130 keys in fp32, so a short
        // cache splits only as far as one block per CU, and never below 256 keys.  A CU given
        // two such blocks runs each at well under half speed: on the 64-node Medusa tree
        // (2048-key cache, 40 row-tile groups), 7 splits of 320 keys (280 blocks) take 15.8 us,
        // 6 of 384 (240 blocks) 13.9 us, 11 of 192 (440 blocks) 16.5 us.
        // Long caches split further, to about four blocks per CU with splits of at least
        // 1024 keys (their blocks otherwise walk thousands of tiles one after another).
        // Measured on random trees with a 16384-key cache, 516 / 1028 / 2052 / 4100 rows:
        // 106.2 / 180.0 / 344.4 / 656.5 us with the short-cache rule, 77.9 / 136.8 / 237.4 /
        // 452.2 us with this one; on a 2048-key cache the short-cache rule stays ahead
        // (516 rows: 27.9 vs 31.6 us).
        const int64_t cus = cu_count;
        const bool long_cache = Tmax > 6144;
        const int64_t target = long_cache ? 4 * cus : cus;
        if (groups >= target) {
            sk = Tmax;
        } else {
            // long caches: at least `target` blocks; short ones: at most one per CU
            const int64_t nsp = long_cache ? (target + groups - 1) / groups : target / groups;
            sk = (Tmax + nsp - 1) / nsp;
        }
        sk = (sk + unit - 1) / unit * unit;
        const int64_t min_sk = long_cache ? 1024 : 256;
        if (sk < min_sk) sk = min_sk;
    }
    if ((Tmax + sk - 1) / sk > kMaxSplits) sk = ((Tmax + kMaxSplits - 1) / kMaxSplits + unit - 1) / unit * unit;
    if (sk > (int64_t)kMaxTiles * kTileKeys) return false;
    p.split_keys = (int)sk;
    const int64_t nsplit = (Tmax + sk - 1) / sk;
    if (nsplit > kMaxSplits) return false;
    p.nsplit = (int)(nsplit < 1 ? 1 : nsplit);
    // The one-row-wave grid is (split, KV head, sequence), split fastest, and the hardware
    // deals workgroup i to XCD i mod 8.  An even split count lines the splits up with the
    // XCDs (with 8 splits, XCD 0 gets every sequence's first split and XCD 7 only the
    // longest sequences' last ones).  An odd grid width gives each XCD one KV head of every
    // (sequence, split); the extra split index is empty and its blocks return at once.
    // Measured on the 64-sequence batch (contexts 512..8192, 1024-key splits): 8 splits
    // 284 us, 9 splits 197 us.
    p.gsplit = (p.variant == 1 && p.nsplit % 2 == 0) ? p.nsplit + 1 : p.nsplit;
    const int64_t blocks = (int64_t)p.kg_pad * p.RT * p.nsplit;
    if (blocks > 0x7fffffff) return false;
    p.blocks = (unsigned)blocks;
    const size_t D = (size_t)d->D;
    // (the one-row-wave grid puts sequences on its third dimension)
    if (p.variant == 1 && d->B > 65535) return false;
    // the counter area every call's workspace starts with (unused here)
    p.cnt_bytes = kCounterBytes;
    // (with one split the kernel stores its output directly; the partial area stays unused)
    const size_t prows = (size_t)p.KG * p.RT * p.nsplit * rows_blk;
    p.o_bytes = align256(prows * D * sizeof(uint16_t));
    p.part_bytes = p.o_bytes + align256(prows * 2 * sizeof(float));
    p.total = p.cnt_bytes + p.part_bytes;
    return true;
}

static sv_status check_attention(const sv_attn_desc *d)
{
    if (!d) return SV_ERR_INVALID_ARG;
    if (d->dtype != SV_F32 && d->dtype != SV_BF16) return SV_ERR_INVALID_ARG;
    if (d->mask != SV_MASK_CAUSAL && d->mask != SV_MASK_TREE) return SV_ERR_INVALID_ARG;
    if (d->B < 0 || d->n_q < 1 || d->Hq < 1 || d->Hkv < 1 || d->D < 1 || d->max_prefix < 0) return SV_ERR_INVALID_ARG;
    if (d->Hq % d->Hkv != 0) return SV_ERR_INVALID_ARG;
    if (!(d->scale > 0.0f)) return SV_ERR_INVALID_ARG;  // also NaN
    if (d->split_keys < 0) return SV_ERR_INVALID_ARG;
    if (!d->q || !d->k || !d->v || !d->prefix_len || !d->out) return SV_ERR_INVALID_ARG;
    if (!d->kv_off && d->kv_sb < 0) return SV_ERR_INVALID_ARG;
    if (d->mask == SV_MASK_TREE && !d->tree_bits) return SV_ERR_INVALID_ARG;
    if (d->q_sb < 0 || d->q_st < 0 || d->q_sh < 0 || d->kv_sh < 0 || d->kv_st < 0 || d->o_sb < 0 || d->o_st < 0 ||
        d->o_sh < 0 || d->tree_sb < 0)
        return SV_ERR_INVALID_ARG;
    if (d->D != 64 && d->D != 128) return SV_ERR_UNSUPPORTED;
    if (d->mask == SV_MASK_TREE && d->n_q > 32768) return SV_ERR_UNSUPPORTED;
    if ((int64_t)d->max_prefix + d->n_q > 0x7fffffffLL) return SV_ERR_UNSUPPORTED;
    if (d->kv_st > (0x7fffffffLL / 32)) return SV_ERR_UNSUPPORTED;  // in-tile byte offsets are 32-bit
    if (d->dtype == SV_BF16) {
        // 16-byte vector access of q, k, v rows; 8-byte stores of out
        const int64_t s16[] = {d->q_sb, d->q_st, d->q_sh, d->kv_sh, d->kv_st, d->kv_off ? 0 : d->kv_sb};
        for (int64_t x : s16)
            if (x % 8) return SV_ERR_UNSUPPORTED;
        if (((uintptr_t)d->q | (uintptr_t)d->k | (uintptr_t)d->v) & 15) return SV_ERR_UNSUPPORTED;
        if ((d->o_sb | d->o_st | d->o_sh) % 4 || ((uintptr_t)d->out & 7)) return SV_ERR_UNSUPPORTED;
    }
    return SV_OK;
}

// Optional measurement events of a call (from the descriptor; NULL when unused).
struct Events {
    hipEvent_t start, stop, call_stop;
};

// A launch of the call; with a start or stop event, through hipExtLaunchKernel, whose events
// take the kernel's own start and end (the times a kernel trace reports).
template <typename K, typename... Args>
static void launch_timed(K kernel, dim3 grid, dim3 block, hipStream_t s, hipEvent_t start, hipEvent_t stop,
                         Args... args)
{
    if (start || stop)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, s, start, stop, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}

template <typename K>
static void launch_main(K kernel, dim3 grid, dim3 block, hipStream_t s, const Events &ev, const AttnArgs &a)
{
    launch_timed(kernel, grid, block, s, ev.start, ev.stop, a);
}

template <int DH, int NWR, int NWK>
static hipError_t launch_variant(const Plan &p, const AttnArgs &a, hipStream_t s, const Events &ev)
{
    if constexpr (NWR == 1) {
        if (p.spec)
            launch_main(attn_bf16_kernel<DH, 1, NWK, true>, dim3(p.gsplit, a.Hkv, a.B), dim3(64 * NWK), s, ev, a);
        else
            launch_main(attn_bf16_kernel<DH, 1, NWK, false>, dim3(p.gsplit, a.Hkv, a.B), dim3(64 * NWK), s, ev, a);
    } else {
        launch_main(attn_bf16_kernel<DH, NWR, NWK, false>, dim3(p.blocks), dim3(64 * NWR * NWK), s, ev, a);
    }
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && p.nsplit == 1 && ev.call_stop) e = hipEventRecord(ev.call_stop, s);
    if (e != hipSuccess || p.nsplit == 1) return e;
    constexpr int ROWS_BLK = 32 * NWR;
    const int tile_rows = p.rows < ROWS_BLK ? p.rows : ROWS_BLK;
    // split lanes per row: one per split up to 8; beyond, each lane takes SPT splits
    int nsl = p.nsplit <= 1 ? 1 : p.nsplit <= 2 ? 2 : p.nsplit <= 4 ? 4 : 8;
    int need = (p.nsplit + nsl - 1) / nsl;
    int spt = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;
    // one float4 per thread while the grid stays small, else four
    const int nrc1 = (tile_rows + kCombThreads / (nsl * (DH / 4)) - 1) / (kCombThreads / (nsl * (DH / 4)));
    const int vpt = (int64_t)nrc1 * p.KG * p.RT > 4 * (p.max_blocks / 16) ? 4 : 1;
    // Large grids: four split lanes per row, each reading two or more splits -- twice the
    // rows per block, so fewer blocks, each waiting once for its sequence length and
    // partials (64-sequence batch, 5 splits: 2560 -> 1536 blocks, combine 10.9 -> 6.6 us;
    // two lanes of four splits: 6.9 us; four lanes with eight float4 columns: 8.4 us)
    if (vpt == 4 && nsl == 8 && p.nsplit <= 32) {
        nsl = 4;
        need = (p.nsplit + nsl - 1) / nsl;
        spt = need <= 2 ? 2 : need <= 4 ? 4 : 8;
    }
    const int cr = kCombThreads / (nsl * (DH / 4 / vpt));      // rows per block
    const int nrc = (tile_rows + cr - 1) / cr;                  // row chunks per tile
    const int ntask = nrc * p.KG * p.RT;
    const int grid = ntask < p.max_blocks ? ntask : p.max_blocks;
    const dim3 g(grid), blk(kCombThreads);
#define SV_COMBINE2(NSL_, SPT_, V_) \
    launch_timed(attn_combine_kernel<DH, ROWS_BLK, NSL_, SPT_, V_>, g, blk, s, nullptr, ev.call_stop, a, nrc, ntask)
#define SV_COMBINE(NSL_, SPT_) \
    do { if (vpt == 1) SV_COMBINE2(NSL_, SPT_, 1); else SV_COMBINE2(NSL_, SPT_, 4); } while (0)
    if (nsl == 1) SV_COMBINE(1, 1);
    else if (nsl == 2) SV_COMBINE(2, 1);
    else if (nsl == 4 && spt == 1) SV_COMBINE(4, 1);
    else if (nsl == 4 && spt == 2) SV_COMBINE(4, 2);
    else if (nsl == 4 && spt == 4) SV_COMBINE(4, 4);
    else if (nsl == 4) SV_COMBINE(4, 8);
    else if (spt == 1) SV_COMBINE(8, 1);
    else if (spt == 2) SV_COMBINE(8, 2);
    else if (spt == 4) SV_COMBINE(8, 4);
    else SV_COMBINE(8, 8);
#undef SV_COMBINE
#undef SV_COMBINE2
    return hipGetLastError();
}

template <int DH>
static hipError_t launch_bf16(const Plan &p, const AttnArgs &a, hipStream_t s, const Events &ev)
{
    switch (p.variant) {
    case 1: return launch_variant<DH, 1, 4>(p, a, s, ev);
    case 2: return launch_variant<DH, 2, 2>(p, a, s, ev);
    default: return launch_variant<DH, 4, 1>(p, a, s, ev);
    }
}

}  // namespace

extern "C" size_t sv_verify_attention_workspace(const sv_attn_desc *d)
{
    if (check_attention(d) != SV_OK) return 0;
    Plan p;
    if (!plan_attention(d, device_cu_count(), p)) return 0;
    return p.total;
}

extern "C" sv_status sv_verify_attention(const sv_attn_desc *d, void *workspace, size_t workspace_bytes, void *stream)
{
    const sv_status st = check_attention(d);
    if (st != SV_OK) return st;
    if (d->B == 0) return SV_OK;
    const int cus = device_cu_count();
    Plan p;
    if (!plan_attention(d, cus, p)) return SV_ERR_UNSUPPORTED;
    if (p.total > 0 && (!workspace || workspace_bytes < p.total || ((uintptr_t)workspace & 255)))
        return SV_ERR_WORKSPACE;

    AttnArgs a;
    a.q = d->q;
    a.q_sb = d->q_sb;
    a.q_st = d->q_st;
    a.q_sh = d->q_sh;
    a.k = d->k;
    a.v = d->v;
    a.kv_off = d->kv_off;
    a.kv_sh = d->kv_sh;
    a.kv_st = d->kv_st;
    a.kv_sb = d->kv_sb;
    a.prefix_len = d->prefix_len;
    a.max_prefix = d->max_prefix;
    a.tmax = d->max_prefix + d->n_q;
    a.tree_bits = d->tree_bits;
    a.tree_sb = d->tree_sb;
    a.words = (d->n_q + 31) / 32;
    a.tree = d->mask == SV_MASK_TREE;
    a.out = d->out;
    a.o_sb = d->o_sb;
    a.o_st = d->o_st;
    a.o_sh = d->o_sh;
    a.lse = d->lse;
    a.B = d->B;
    a.n_q = d->n_q;
    a.Hq = d->Hq;
    a.Hkv = d->Hkv;
    a.G = d->Hq / d->Hkv;
    a.rows = p.rows;
    a.RT = p.RT;
    a.KG = p.KG;
    a.nsplit = p.nsplit;
    a.split_keys = p.split_keys;
    a.scale_log2 = d->scale * kLog2e;
    a.part = p.part_bytes ? (float *)((char *)workspace + p.cnt_bytes) : nullptr;
    a.pml = p.part_bytes ? (float2 *)((char *)workspace + p.cnt_bytes + p.o_bytes) : nullptr;

    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    hipError_t e;
    if (p.variant == 0) {
        const int64_t nrows = (int64_t)d->B * d->n_q * d->Hq;
        if (nrows > 0x7fffffffLL) return SV_ERR_UNSUPPORTED;
        hipLaunchKernelGGL(attn_f32_kernel, dim3((unsigned)nrows), dim3(64), 0, s, a, d->D);
        e = hipGetLastError();
    } else {
        p.max_blocks = 16 * cus;
        // A grid of at most one block per CU is latency-bound: with a dense cache layout
        // (no kv_off) the first tiles are loaded while the sequence lengths are in flight.
        // Larger grids skip it (their empty splits would load tiles for nothing).
        p.spec = p.variant == 1 && !d->kv_off && (int64_t)p.gsplit * d->Hkv * d->B <= cus;
        const Events ev{(hipEvent_t)d->ev_kernel_start, (hipEvent_t)d->ev_kernel_stop, (hipEvent_t)d->ev_call_stop};
        e = d->D == 128 ? launch_bf16<128>(p, a, s, ev) : launch_bf16<64>(p, a, s, ev);
    }
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}
