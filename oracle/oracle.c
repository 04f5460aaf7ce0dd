/*
 * oracle.c -- plain, slow, fp64 CPU oracle for the speculative-decoding verify step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or helper with the HIP library under
 * draft_token_verification_attention_amd/, and neither side includes the other.
 *
 * Sources (the pages this follows, cited by title and section):
 *   [TB]  "Speculative decoding", Zero to Frontier textbook, chapter 20, section 20.5.
 *   [MED] "Speculative-Decoding" (s1mplewind blog, Medusa reading notes).
 *   [AG]  "Speculative Decoding: The Art of Guessing Well" (astralord blog).
 *   [PHX] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11
 *         (the Philox4x64-10 generator; the pages name no generator).
 *
 * Every floating-point quantity is computed in double precision.  Logits arrive
 * as fp32 and attention inputs as fp32 or bf16; both widen exactly to double.
 * Loops are the definitions written out: no blocking, no fusion, no reordering
 * beyond what the definition states.  OpenMP is used only across independent
 * outputs (sequences, attention rows); it never splits a single sum.
 *
 * Pins: every function here is pinned by tests in tests/test_oracle_*.py
 * against values the pages print, closed forms, library routines and brute force.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------------- */
/* Philox4x64-10 [PHX].  A counter-based generator: block = f_key(counter).   */
/* Round: two 64x64->128 products of counter words 0 and 2 with fixed          */
/* multipliers, XOR-mixed with the other words and the key; the key is bumped  */
/* by two Weyl constants between rounds.  Constants are the published ones.    */
/* ------------------------------------------------------------------------- */
static const uint64_t PHX_M0 = 0xD2E7470EE14C6C93ULL;
static const uint64_t PHX_M1 = 0xCA5A826395121157ULL;
static const uint64_t PHX_W0 = 0x9E3779B97F4A7C15ULL; /* golden ratio */
static const uint64_t PHX_W1 = 0xBB67AE8584CAA73BULL; /* sqrt(3) - 1 */

ORC_EXPORT void orc_philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4])
{
    uint64_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        unsigned __int128 p0 = (unsigned __int128)PHX_M0 * c0;
        unsigned __int128 p1 = (unsigned __int128)PHX_M1 * c2;
        uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
        uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
        uint64_t n0 = hi1 ^ c1 ^ k0;
        uint64_t n1 = lo1;
        uint64_t n2 = hi0 ^ c3 ^ k1;
        uint64_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += PHX_W0;
        k1 += PHX_W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Uniform on (0,1) from the first output word: (2*(w0>>12)+1) * 2^-53.
 * Every value is exact in double, never 0 and never 1.
 * Counter = (c0, step, stream, tag), key = (seed, 0).                          */
ORC_EXPORT double orc_uniform(uint64_t seed, uint64_t c0, uint64_t step, uint64_t stream, uint64_t tag)
{
    uint64_t ctr[4] = {c0, step, stream, tag};
    uint64_t key[2] = {seed, 0};
    uint64_t out[4];
    orc_philox4x64_10(ctr, key, out);
    return (double)(2 * (out[0] >> 12) + 1) * 0x1p-53;
}

#define ORC_TAG_ACCEPT 0x53560001ULL
#define ORC_TAG_WALK   0x53560002ULL
/* Near-threshold windows.  A ratio test is near when |u - p/q| < 1e-6 (the tolerance
 * of accept decisions).  A draw u*Z from weights in units of probability mass
 * (p, or the residual (p - q)+ with p, q normalized) is near when it lies within 1e-10 of
 * either cumulative sum that brackets the chosen token: the fp64 sums over a 128K-token row
 * are exact to about 1e-11, so a draw farther away than this is decided by the arithmetic
 * alone.  (A window of 1e-6 Z flagged a sixth of all draws at 128K tokens.)              */
#define ORC_NEAR_RATIO 1e-6
#define ORC_NEAR_DRAW  1e-10

/* ------------------------------------------------------------------------- */
/* Token tree -> ancestor-or-self mask, depth and position ids.               */
/* [TB] section "Token trees check several guesses at once", box "Token tree  */
/* and tree attention", and the exercise "The tree attention mask": par(i) is  */
/* -1 or an earlier node; node i sees every prefix position, itself and its    */
/* ancestors; depth = number of ancestors; position id = P + depth.            */
/* bits: n rows of `words` uint32; bit (j%32) of word j/32 of row i is set iff */
/* j == i or j is an ancestor of i.  Returns 0, or 1 + the first bad node.     */
/* ------------------------------------------------------------------------- */
ORC_EXPORT int32_t orc_tree_mask(const int32_t *parents, int32_t n, int32_t prefix_len,
                                 uint32_t *bits, int32_t words, int32_t *depth, int64_t *pos)
{
    for (int32_t i = 0; i < n; ++i)
        if (parents[i] < -1 || parents[i] >= i) return i + 1;
    for (int32_t i = 0; i < n; ++i) {
        depth[i] = parents[i] < 0 ? 0 : depth[parents[i]] + 1;
        pos[i] = (int64_t)prefix_len + depth[i];
        uint32_t *row = bits + (int64_t)i * words;
        for (int32_t w = 0; w < words; ++w) row[w] = 0;
        for (int32_t j = i; j >= 0; j = parents[j])      /* self, then each ancestor */
            row[j >> 5] |= 1u << (j & 31);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Verify attention, fp64.                                                    */
/* [TB] section "Checking several tokens costs about as much as writing one": */
/* each new token attends to the whole cache and to the new tokens before it   */
/* (a causal mask aligned to the bottom-right corner).  Trees: box "Token tree */
/* and tree attention" -- every prefix position plus ancestors-or-self.        */
/* Query head h reads KV head h / G with G = Hq / Hkv (grouped queries).       */
/* Softmax: s_j = scale*<q,k_j>, m = max s, w = exp(s - m),                    */
/* o = sum w v / sum w, lse = m + log(sum w).                                  */
/* dtype: 0 = fp32, 1 = bf16 (raw 16-bit patterns; widened exactly).           */
/* Rows: a list of (b, i, h) triples; out is [n_rows][D], lse [n_rows].        */
/* ------------------------------------------------------------------------- */
static double widen(const void *base, int dtype, int64_t idx)
{
    if (dtype == 0) return (double)((const float *)base)[idx];
    uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

ORC_EXPORT int32_t orc_attention(int32_t dtype, int32_t B, int32_t n_q, int32_t Hq, int32_t Hkv, int32_t D,
                                 double scale, int32_t tree,
                                 const void *q, int64_t q_sb, int64_t q_st, int64_t q_sh,
                                 const void *k, const void *v, const int64_t *kv_off,
                                 int64_t kv_sh, int64_t kv_st,
                                 const int32_t *prefix_len,
                                 const uint32_t *tree_bits, int64_t tree_sb, int32_t words,
                                 const int32_t *rows, int64_t n_rows,
                                 double *out, double *lse)
{
    if (Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || n_q <= 0) return 1;
    const int32_t G = Hq / Hkv;
    int32_t bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int32_t b = rows[3 * r], i = rows[3 * r + 1], h = rows[3 * r + 2];
        if (b < 0 || b >= B || i < 0 || i >= n_q || h < 0 || h >= Hq) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        const int32_t g = h / G;
        const int64_t P = prefix_len[b];
        const int64_t nkeys = P + n_q;
        const int64_t qbase = (int64_t)b * q_sb + (int64_t)i * q_st + (int64_t)h * q_sh;
        const int64_t kvbase = kv_off[b] + (int64_t)g * kv_sh;
        const uint32_t *mrow = tree ? tree_bits + (int64_t)b * tree_sb + (int64_t)i * words : NULL;
        double *o = out + r * D;
        double *s = (double *)malloc(sizeof(double) * (size_t)nkeys);
        char *vis = (char *)malloc((size_t)nkeys);
        double m = -INFINITY;
        for (int64_t t = 0; t < nkeys; ++t) {
            int visible;
            if (t < P) visible = 1;
            else {
                int64_t j = t - P;
                visible = tree ? (int)((mrow[j >> 5] >> (j & 31)) & 1u) : (j <= i);
            }
            vis[t] = (char)visible;
            if (!visible) continue;
            double dot = 0.0;
            for (int32_t d = 0; d < D; ++d)
                dot += widen(q, dtype, qbase + d) * widen(k, dtype, kvbase + t * kv_st + d);
            s[t] = scale * dot;
            if (s[t] > m) m = s[t];
        }
        double l = 0.0;
        for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
        for (int64_t t = 0; t < nkeys; ++t) {
            if (!vis[t]) continue;
            double w = exp(s[t] - m);
            l += w;
            for (int32_t d = 0; d < D; ++d) o[d] += w * widen(v, dtype, kvbase + t * kv_st + d);
        }
        for (int32_t d = 0; d < D; ++d) o[d] /= l;
        if (lse) lse[r] = m + log(l);
        free(s);
        free(vis);
    }
    return bad ? 2 : 0;
}

/* ------------------------------------------------------------------------- */
/* Temperature softmax of one fp32 logit row, in double:                      */
/* p(x) = exp((l(x) - max l)/tau) / sum_x' exp((l(x') - max l)/tau).          */
/* [TB] section "When the target samples...": both models sample at the same  */
/* temperature tau; tau -> 0 is the argmax.                                    */
/* ------------------------------------------------------------------------- */
static void softmax_row(const float *logits, int32_t V, double tau, double *p)
{
    double m = -INFINITY;
    for (int32_t x = 0; x < V; ++x) if ((double)logits[x] > m) m = (double)logits[x];
    double z = 0.0;
    for (int32_t x = 0; x < V; ++x) { p[x] = exp(((double)logits[x] - m) / tau); z += p[x]; }
    for (int32_t x = 0; x < V; ++x) p[x] /= z;
}

/* First index of the largest raw logit (ties go to the lowest token id).     */
static int32_t argmax_row(const float *logits, int32_t V)
{
    int32_t best = 0;
    for (int32_t x = 1; x < V; ++x) if (logits[x] > logits[best]) best = x;
    return best;
}

/* Inverse CDF in ascending token-id order: the smallest y with C_y > u * Z,
 * C the running sum of w, Z the total.  *near is set when u*Z lies within
 * ORC_NEAR_DRAW of C_{y-1} or C_y (a draw whose token could flip under rounding).
 * Returns -1 when Z is not positive.                                          */
static int32_t inverse_cdf(const double *w, int32_t V, double u, int32_t *near)
{
    double z = 0.0;
    for (int32_t x = 0; x < V; ++x) z += w[x];
    if (!(z > 0.0)) return -1;
    const double target = u * z;
    double c = 0.0, prev = 0.0;
    int32_t y = -1;
    for (int32_t x = 0; x < V; ++x) {
        prev = c;
        c += w[x];
        if (c > target) { y = x; break; }
    }
    if (y < 0) { /* rounding left the total just below u*Z: take the last token with mass */
        for (int32_t x = V - 1; x >= 0; --x) if (w[x] > 0.0) { y = x; break; }
        prev = c;
    }
    if (near) *near = (fabs(target - prev) < ORC_NEAR_DRAW) || (fabs(c - target) < ORC_NEAR_DRAW);
    return y;
}

/* ------------------------------------------------------------------------- */
/* Acceptance of one round, per sequence.                                     */
/*                                                                             */
/* GREEDY (mode 0) -- [TB] box "A round of greedy speculative decoding":       */
/*   z_i = argmax of target row i (raw logits; ties -> lowest id),             */
/*   J = number of leading drafts with x_i == z_i, emit x_1..x_J then z_{J+1}. */
/*   Draft logits are not read and no uniform is drawn.                        */
/*                                                                             */
/* SAMPLE (mode 1) -- [TB] box "A round of speculative sampling" and box       */
/* "The speculative sampling rule"; [AG] section "Speculative sampling":       */
/*   p_i = softmax(target_i / tau), q_i = softmax(draft_i / tau);             */
/*   for i = 0..gamma-1 in order, u_i = U(seed; i, step, stream, ACCEPT);      */
/*   accept x_i iff u_i * q_i(x_i) < p_i(x_i) (u < p/q written without a       */
/*   division; a token with q = 0 is never drafted, and then the test passes   */
/*   iff p > 0); stop at the first failure; J = number accepted.               */
/*   The extra token is drawn from r = max(0, p_J - q_J), or from p_gamma     */
/*   when J = gamma (a zero draft row after the last draft, as in the          */
/*   "Speculative verification in PyTorch" section), by inverse CDF with the   */
/*   dedicated uniform u* = U(seed; gamma, step, stream, ACCEPT).              */
/*   A zero residual (impossible in exact arithmetic after a rejection) falls  */
/*   back to p_J.                                                              */
/* tau == 0 in SAMPLE mode is treated as GREEDY ([TB]: tau -> 0 is greedy).    */
/*                                                                             */
/* Outputs: accept_len[B]; out_tokens[B][gamma+1] (J drafts, the extra token,  */
/* then -1); alpha[B][gamma] = sum_x min(p_i, q_i) when non-null (SAMPLE);     */
/* flags[B]: bit0 = an evaluated ratio test had |u - p/q| < 1e-6,              */
/* bit1 = the extra draw lay within 1e-10 of a CDF boundary.                   */
/* ------------------------------------------------------------------------- */
ORC_EXPORT int32_t orc_spec_accept(int32_t mode, int32_t B, int32_t gamma, int32_t V, float temperature,
                                   const float *target, const float *draft, const int32_t *draft_tokens,
                                   uint64_t seed, uint64_t step, const uint64_t *stream_ids,
                                   int32_t *accept_len, int32_t *out_tokens, double *alpha, int32_t *flags)
{
    if (B < 0 || gamma < 0 || V <= 0) return 1;
    const int greedy = (mode == 0) || (temperature == 0.0f);
    const double tau = (double)temperature;
    int32_t bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t b = 0; b < B; ++b) {
        const float *tb = target + (int64_t)b * (gamma + 1) * V;
        const int32_t *xb = draft_tokens + (int64_t)b * gamma;
        int32_t *ob = out_tokens + (int64_t)b * (gamma + 1);
        int32_t fl = 0;
        for (int32_t i = 0; i < gamma; ++i)
            if (xb[i] < 0 || xb[i] >= V) {
#pragma omp atomic write
                bad = 1;
            }
        for (int32_t i = 0; i <= gamma; ++i) ob[i] = -1;
        if (greedy) {
            int32_t J = 0;
            while (J < gamma && xb[J] == argmax_row(tb + (int64_t)J * V, V)) ++J;
            for (int32_t i = 0; i < J; ++i) ob[i] = xb[i];
            ob[J] = argmax_row(tb + (int64_t)J * V, V);
            accept_len[b] = J;
            if (flags) flags[b] = 0;
            if (alpha) for (int32_t i = 0; i < gamma; ++i) alpha[(int64_t)b * gamma + i] = NAN;
            continue;
        }
        const float *db = draft + (int64_t)b * gamma * V;
        const uint64_t stream = stream_ids ? stream_ids[b] : (uint64_t)b;
        double *p = (double *)malloc(sizeof(double) * (size_t)V);
        double *q = (double *)malloc(sizeof(double) * (size_t)V);
        if (alpha) {
            for (int32_t i = 0; i < gamma; ++i) {
                softmax_row(tb + (int64_t)i * V, V, tau, p);
                softmax_row(db + (int64_t)i * V, V, tau, q);
                double a = 0.0;
                for (int32_t x = 0; x < V; ++x) a += fmin(p[x], q[x]);
                alpha[(int64_t)b * gamma + i] = a;
            }
        }
        int32_t J = 0;
        for (; J < gamma; ++J) {
            softmax_row(tb + (int64_t)J * V, V, tau, p);
            softmax_row(db + (int64_t)J * V, V, tau, q);
            const int32_t x = xb[J];
            const double u = orc_uniform(seed, (uint64_t)J, step, stream, ORC_TAG_ACCEPT);
            const double px = p[x], qx = q[x];
            if (qx > 0.0 && fabs(u - px / qx) < ORC_NEAR_RATIO) fl |= 1;
            if (!(u * qx < px)) break;
        }
        /* the extra token */
        softmax_row(tb + (int64_t)J * V, V, tau, p);
        if (J < gamma) {
            softmax_row(db + (int64_t)J * V, V, tau, q);
            for (int32_t x = 0; x < V; ++x) q[x] = fmax(0.0, p[x] - q[x]);
        } else {
            memcpy(q, p, sizeof(double) * (size_t)V);
        }
        const double ustar = orc_uniform(seed, (uint64_t)gamma, step, stream, ORC_TAG_ACCEPT);
        int32_t near = 0;
        int32_t y = inverse_cdf(q, V, ustar, &near);
        if (y < 0) y = inverse_cdf(p, V, ustar, &near);
        if (near) fl |= 2;
        for (int32_t i = 0; i < J; ++i) ob[i] = xb[i];
        ob[J] = y;
        accept_len[b] = J;
        if (flags) flags[b] = fl;
        free(p);
        free(q);
    }
    return bad ? 2 : 0;
}

/* ------------------------------------------------------------------------- */
/* Tree walk, per sequence.                                                   */
/* Node 0 is the root (the last committed token, parent -1); logits row v is   */
/* the target's next-token distribution after node v.  Starting at v = 0, for  */
/* d = 0, 1, ...: y = argmax of row v (GREEDY) or an inverse-CDF draw from     */
/* softmax(row v / tau) with u = U(seed; d, step, stream, WALK) (SAMPLE);      */
/* move to the first child of v (in node order) whose token is y; when there   */
/* is none, emit y and stop.                                                   */
/* GREEDY: [TB] section "Token trees check several guesses at once" (the walk  */
/* after the mask exercise).  SAMPLE: [MED] section "Attention Tree" -- sample */
/* from the target at the node, look for that token among the children, and    */
/* go down level by level until no child matches.                              */
/* Outputs: accept_len[B] = J; path[B][max_depth+1] = (0, n_1, ..., n_J, -1..);*/
/* out_tokens[B][max_depth+1] = (tokens of n_1..n_J, y, -1..); flags[B] bit1   */
/* = some draw lay within 1e-10 of a CDF boundary.                             */
/* Returns 0; 3 if a walk would pass max_depth (that walk stops at the node  */
/* at depth max_depth and emits its choice y); 2 on a bad token/parent.       */
/* ------------------------------------------------------------------------- */
ORC_EXPORT int32_t orc_tree_walk(int32_t mode, int32_t B, int32_t n, int32_t V, int32_t max_depth,
                                 float temperature, const float *logits, const int32_t *tokens,
                                 const int32_t *parents, uint64_t seed, uint64_t step,
                                 const uint64_t *stream_ids, int32_t *accept_len, int32_t *path,
                                 int32_t *out_tokens, int32_t *flags)
{
    if (B < 0 || n <= 0 || V <= 0 || max_depth < 0) return 1;
    if (parents[0] != -1) return 2;
    for (int32_t i = 1; i < n; ++i) if (parents[i] < -1 || parents[i] >= i) return 2;
    const int greedy = (mode == 0) || (temperature == 0.0f);
    const double tau = (double)temperature;
    int32_t status = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t b = 0; b < B; ++b) {
        const float *lb = logits + (int64_t)b * n * V;
        const int32_t *tk = tokens + (int64_t)b * n;
        int32_t *pb = path + (int64_t)b * (max_depth + 1);
        int32_t *ob = out_tokens + (int64_t)b * (max_depth + 1);
        const uint64_t stream = stream_ids ? stream_ids[b] : (uint64_t)b;
        double *p = greedy ? NULL : (double *)malloc(sizeof(double) * (size_t)V);
        for (int32_t d = 0; d <= max_depth; ++d) { pb[d] = -1; ob[d] = -1; }
        int32_t fl = 0, v = 0, d = 0;
        pb[0] = 0;
        for (;;) {
            const float *row = lb + (int64_t)v * V;
            int32_t y;
            if (greedy) y = argmax_row(row, V);
            else {
                softmax_row(row, V, tau, p);
                int32_t near = 0;
                y = inverse_cdf(p, V, orc_uniform(seed, (uint64_t)d, step, stream, ORC_TAG_WALK), &near);
                if (near) fl |= 2;
            }
            int32_t child = -1;
            for (int32_t c = v + 1; c < n; ++c)
                if (parents[c] == v && tk[c] == y) { child = c; break; }
            if (child < 0) { ob[d] = y; break; }
            if (d + 1 > max_depth) {   /* no room below: the choice at v is emitted */
#pragma omp atomic write
                status = 3;
                ob[d] = y;
                break;
            }
            ob[d] = tk[child];
            v = child;
            ++d;
            pb[d] = child;
        }
        accept_len[b] = d;
        if (flags) flags[b] = fl;
        free(p);
    }
    return status;
}

/* ========================================================================= */
/* Beyond the verify step proper: the cache commit after a round, and three   */
/* other verification rules the pages give.                                  */
/* ========================================================================= */

#define ORC_TAG_GUMBEL 0x53560003ULL
#define ORC_TAG_RRS    0x53560004ULL
#define ORC_NEAR_GUMBEL 1e-12

/* ------------------------------------------------------------------------- */
/* KV-cache commit.  [TB] section "Keeping the caches consistent after a      */
/* rejection": after J acceptances the entries of the accepted drafts are      */
/* right and those of the rejected ones are discarded; the correction or bonus */
/* token has no entry yet.  A contiguous cache rolls back by moving its length */
/* pointer; a tree needs one more step, gathering the accepted branch's        */
/* entries (scattered among discarded siblings) into consecutive slots.  [AG]  */
/* section "Verification bottlenecks" (KV cache bookkeeping) says the same.    */
/* The pass wrote node j (chain row j) of sequence b at position P_b + j, node */
/* 0 being the last committed token.  Afterwards position P_b + k holds the    */
/* entry of path node k, k = 1..J, and the length is P_b + 1 + J.  Element    */
/* (t, g, d) of a cache is at kv_off[b] + g kv_sh + t kv_st + d, esize bytes.  */
/* path == NULL: a chain, only the length moves.  Returns 0, or 1 + the first  */
/* sequence with J or a path node out of range (that sequence is untouched).   */
/* ------------------------------------------------------------------------- */
ORC_EXPORT int32_t orc_kv_commit(int32_t B, int32_t n_q, int32_t Hkv, int32_t D, int32_t esize,
                                 void *k, void *v, const int64_t *kv_off, int64_t kv_sh, int64_t kv_st,
                                 const int32_t *prefix_len, const int32_t *accept_len,
                                 const int32_t *path, int32_t path_stride, int32_t *new_len)
{
    int32_t bad = 0;
    for (int32_t b = 0; b < B; ++b) {
        const int64_t P = prefix_len[b];
        const int32_t J = accept_len[b];
        new_len[b] = prefix_len[b];
        int ok = (J >= 0 && J < n_q);
        if (ok && path)
            for (int32_t kk = 1; kk <= J; ++kk) {
                const int32_t node = path[(int64_t)b * path_stride + kk];
                if (node < kk || node >= n_q) ok = 0;
            }
        if (!ok) {
            if (!bad) bad = b + 1;
            continue;
        }
        if (path) {
            for (int32_t kk = 1; kk <= J; ++kk) {       /* in path order: a slot is written */
                const int32_t node = path[(int64_t)b * path_stride + kk];  /* after it was read */
                if (node == kk) continue;
                for (int32_t g = 0; g < Hkv; ++g) {
                    const int64_t src = kv_off[b] + g * kv_sh + (P + node) * kv_st;
                    const int64_t dst = kv_off[b] + g * kv_sh + (P + kk) * kv_st;
                    memcpy((char *)k + dst * esize, (char *)k + src * esize, (size_t)D * esize);
                    memcpy((char *)v + dst * esize, (char *)v + src * esize, (size_t)D * esize);
                }
            }
        }
        new_len[b] = (int32_t)(P + 1 + J);
    }
    return bad;
}

/* ------------------------------------------------------------------------- */
/* Block verification.  [AG] section "Block verification": with p_k, q_k the  */
/* target's and drafter's distributions at draft position k (target row k-1,  */
/* draft row k-1 here) and x_k the k-th draft, the running weight             */
/*   w_0 = 1,  w_k = min(1, w_{k-1} p_k(x_k) / q_k(x_k));                      */
/* prefix k survives with probability                                         */
/*   h_k = m_k / (m_k + 1 - w_k) (1 when w_k = 1),                             */
/*   m_k = sum_x (w_k p_{k+1}(x) - q_{k+1}(x))+,  q_{gamma+1} = 0 (m_gamma = w_gamma);*/
/* the longest surviving prefix n is kept and the next token is drawn from    */
/* (w_n p_{n+1} - q_{n+1})+ normalized.  Uniforms: survival of prefix k uses  */
/* index k-1, the draw index gamma (tag ACCEPT, as speculative sampling: with */
/* gamma = 1 the two rules take the same decisions).  A drafted token with    */
/* q = 0 sets w_k = 1 if p > 0 (and w_{k-1} > 0), else 0.  A zero residual     */
/* falls back to p_{n+1}.  p, q = softmax(logits / T).                         */
/* gamma = 0 (no draft verified): one draw from p_1 with the uniform of index */
/* 0, as in orc_spec_accept.                                                  */
/* Outputs as orc_spec_accept; weights[B][gamma+1] = w_0..w_gamma (optional);  */
/* flags bit0 = some |u - h_k| < 1e-6, bit1 = the draw within 1e-10 of a      */
/* CDF boundary.                                                              */
/* ------------------------------------------------------------------------- */
ORC_EXPORT int32_t orc_block_accept(int32_t B, int32_t gamma, int32_t V, float temperature,
                                    const float *target, const float *draft, const int32_t *draft_tokens,
                                    uint64_t seed, uint64_t step, const uint64_t *stream_ids,
                                    int32_t *accept_len, int32_t *out_tokens, double *weights, int32_t *flags)
{
    if (B < 0 || gamma < 0 || V <= 0 || !(temperature > 0.0f)) return 1;
    const double tau = (double)temperature;
    int32_t bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t b = 0; b < B; ++b) {
        const float *tb = target + (int64_t)b * (gamma + 1) * V;
        const float *db = draft + (int64_t)b * gamma * V;
        const int32_t *xb = draft_tokens + (int64_t)b * gamma;
        int32_t *ob = out_tokens + (int64_t)b * (gamma + 1);
        const uint64_t stream = stream_ids ? stream_ids[b] : (uint64_t)b;
        double *p = (double *)malloc(sizeof(double) * (size_t)V);
        double *q = (double *)malloc(sizeof(double) * (size_t)V);
        double *w = (double *)malloc(sizeof(double) * (size_t)(gamma + 1));
        int32_t fl = 0, n = 0;
        for (int32_t i = 0; i <= gamma; ++i) ob[i] = -1;
        for (int32_t i = 0; i < gamma; ++i)
            if (xb[i] < 0 || xb[i] >= V) {
#pragma omp atomic write
                bad = 1;
            }
        w[0] = 1.0;
        for (int32_t kk = 1; kk <= gamma; ++kk) {
            const int32_t x = xb[kk - 1];
            softmax_row(tb + (int64_t)(kk - 1) * V, V, tau, p);
            softmax_row(db + (int64_t)(kk - 1) * V, V, tau, q);
            if (q[x] > 0.0) w[kk] = fmin(1.0, w[kk - 1] * p[x] / q[x]);
            else w[kk] = (w[kk - 1] > 0.0 && p[x] > 0.0) ? 1.0 : 0.0;
        }
        for (int32_t kk = 1; kk <= gamma; ++kk) {
            double m;
            if (kk < gamma) {
                softmax_row(tb + (int64_t)kk * V, V, tau, p);
                softmax_row(db + (int64_t)kk * V, V, tau, q);
                m = 0.0;
                for (int32_t x = 0; x < V; ++x) m += fmax(0.0, w[kk] * p[x] - q[x]);
            } else {
                m = w[gamma];
            }
            const double h = w[kk] < 1.0 ? m / (m + 1.0 - w[kk]) : 1.0;
            const double u = orc_uniform(seed, (uint64_t)(kk - 1), step, stream, ORC_TAG_ACCEPT);
            if (fabs(u - h) < ORC_NEAR_RATIO) fl |= 1;
            if (u <= h) n = kk;
        }
        /* the next token, from (w_n p_{n+1} - q_{n+1})+ */
        softmax_row(tb + (int64_t)n * V, V, tau, p);
        if (n < gamma) {
            softmax_row(db + (int64_t)n * V, V, tau, q);
            for (int32_t x = 0; x < V; ++x) q[x] = fmax(0.0, w[n] * p[x] - q[x]);
        } else {
            for (int32_t x = 0; x < V; ++x) q[x] = w[gamma] * p[x];
        }
        const double ustar = orc_uniform(seed, (uint64_t)gamma, step, stream, ORC_TAG_ACCEPT);
        int32_t near = 0;
        int32_t y = inverse_cdf(q, V, ustar, &near);
        if (y < 0) y = inverse_cdf(p, V, ustar, &near);
        if (near) fl |= 2;
        for (int32_t i = 0; i < n; ++i) ob[i] = xb[i];
        ob[n] = y;
        accept_len[b] = n;
        if (weights)
            for (int32_t i = 0; i <= gamma; ++i) weights[(int64_t)b * (gamma + 1) + i] = w[i];
        if (flags) flags[b] = fl;
        free(p);
        free(q);
        free(w);
    }
    return bad ? 2 : 0;
}

/* ------------------------------------------------------------------------- */
/* Gumbel-max with shared noise.  [AG] section "Sampling with shared noise":  */
/* sampling from softmax(l) is argmax_x (l(x) + g_x), g_x = -log(-log u_x);   */
/* drafter and target share the noise vector g_i of draft position i.         */
/* Here l = logits / T, and u_x of position i is word (x mod 4) of the Philox */
/* block with counter (x div 4, step, stream, TAG_GUMBEL + 2^32 i), mapped to */
/* (0,1) like every uniform.  T = 0: the plain argmax (no noise).  Ties go to */
/* the lowest token.  gap = best score - second best (+inf when V = 1).        */
/* ------------------------------------------------------------------------- */
static int32_t gumbel_argmax_row(const float *logits, int32_t V, double tau, uint64_t seed, uint64_t step,
                                 uint64_t stream, uint64_t pos, double *gap)
{
    double best = -INFINITY, second = -INFINITY;
    int32_t arg = 0;
    uint64_t words[4] = {0, 0, 0, 0};
    for (int32_t x = 0; x < V; ++x) {
        double s;
        if (tau == 0.0) {
            s = (double)logits[x];
        } else {
            if ((x & 3) == 0) {
                uint64_t ctr[4] = {(uint64_t)x >> 2, step, stream, ORC_TAG_GUMBEL + (pos << 32)};
                uint64_t key[2] = {seed, 0};
                orc_philox4x64_10(ctr, key, words);
            }
            const double u = (double)(2 * (words[x & 3] >> 12) + 1) * 0x1p-53;
            s = (double)logits[x] / tau + (-log(-log(u)));
        }
        if (s > best) {
            second = best;
            best = s;
            arg = x;
        } else if (s > second) {
            second = s;
        }
    }
    if (gap) *gap = best - second;
    return arg;
}

/* argmax_x (l_{b,i}(x) / T + g_{i,x}) for every row i of `rows` rows per sequence    */
/* (position i): the target's own samples, or the drafter's proposals when given   */
/* the drafter's logits.  out [B][rows]; gap [B][rows] optional.                    */
ORC_EXPORT int32_t orc_gumbel_argmax(int32_t B, int32_t rows, int32_t V, float temperature, const float *logits,
                                     uint64_t seed, uint64_t step, const uint64_t *stream_ids, int32_t *out,
                                     double *gap)
{
    if (B < 0 || rows < 0 || V <= 0 || !(temperature >= 0.0f)) return 1;
    const double tau = (double)temperature;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t b = 0; b < B; ++b) {
        const uint64_t stream = stream_ids ? stream_ids[b] : (uint64_t)b;
        for (int32_t i = 0; i < rows; ++i)
            out[(int64_t)b * rows + i] = gumbel_argmax_row(logits + ((int64_t)b * rows + i) * V, V, tau, seed,
                                                           step, stream, (uint64_t)i,
                                                           gap ? gap + (int64_t)b * rows + i : NULL);
    }
    return 0;
}

/* Gumbel-coupled verification ([AG], same section): the target's sample y_i  */
/* at every position, the longest prefix with x_i == y_i is kept (J), and y_J */
/* is appended -- exact matching, as under greedy decoding; the output is what */
/* the target samples with that noise on its own (gamma = 0: just y_0).      */
/* Outputs as orc_spec_accept;                                                 */
/* flags bit0 = an evaluated position's best two scores within 1e-12.          */
ORC_EXPORT int32_t orc_gumbel_accept(int32_t B, int32_t gamma, int32_t V, float temperature, const float *target,
                                     const int32_t *draft_tokens, uint64_t seed, uint64_t step,
                                     const uint64_t *stream_ids, int32_t *accept_len, int32_t *out_tokens,
                                     int32_t *flags)
{
    if (B < 0 || gamma < 0 || V <= 0 || !(temperature >= 0.0f)) return 1;
    const double tau = (double)temperature;
    int32_t bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t b = 0; b < B; ++b) {
        const float *tb = target + (int64_t)b * (gamma + 1) * V;
        const int32_t *xb = draft_tokens + (int64_t)b * gamma;
        int32_t *ob = out_tokens + (int64_t)b * (gamma + 1);
        const uint64_t stream = stream_ids ? stream_ids[b] : (uint64_t)b;
        int32_t fl = 0, J = 0, y = -1;
        for (int32_t i = 0; i <= gamma; ++i) ob[i] = -1;
        for (int32_t i = 0; i < gamma; ++i)
            if (xb[i] < 0 || xb[i] >= V) {
#pragma omp atomic write
                bad = 1;
            }
        for (;;) {
            double gap;
            y = gumbel_argmax_row(tb + (int64_t)J * V, V, tau, seed, step, stream, (uint64_t)J, &gap);
            if (gap < ORC_NEAR_GUMBEL) fl |= 1;
            if (J == gamma || xb[J] != y) break;
            ob[J] = y;
            ++J;
        }
        ob[J] = y;
        accept_len[b] = J;
        if (flags) flags[b] = fl;
    }
    return bad ? 2 : 0;
}

/* ------------------------------------------------------------------------- */
/* Tree verification by recursive rejection.  [TB] box "Recursive rejection   */
/* at a node with several children": the children s_1..s_k of a node (node    */
/* order) were drawn from the drafter's q at that node; with R_1 = p, try     */
/* s_i: accept with probability min(1, R_i(s_i)/q(s_i)) and move to that      */
/* child; on rejection R_{i+1} = (R_i - q)+ normalized.  If every child is    */
/* rejected (or the node is a leaf), the extra token is drawn from R_{k+1}.    */
/* without_replacement: the children were drawn without replacement (the     */
/* Sequoia variant the same section describes): after a rejection the        */
/* rejected token is also zeroed in q and q renormalized.                     */
/* p, q = softmax(target / T), softmax(draft / T) of the node's rows (row v   */
/* of the drafter's logits is the distribution it drew v's children from).   */
/* Uniforms (tag RRS): try i at depth d uses index 2^16 d + i, the draw       */
/* 2^16 d + 0xffff.  Accept test u q(s) < R(s) (as u < R/q; q(s) = 0 passes   */
/* iff R(s) > 0).  A zero (R - q)+ (rounding only) keeps R.  At max_depth an   */
/* accepted child's token is emitted as the extra token (status 3).           */
/* Outputs as orc_tree_walk; flags bit0 = a test with |u - R/q| < 1e-6, bit1 = */
/* the draw within 1e-10 of a CDF boundary.                                   */
/* ------------------------------------------------------------------------- */
ORC_EXPORT int32_t orc_tree_rrs(int32_t B, int32_t n, int32_t V, int32_t max_depth, float temperature,
                                int32_t without_replacement, const float *target, const float *draft,
                                const int32_t *tokens, const int32_t *parents, uint64_t seed, uint64_t step,
                                const uint64_t *stream_ids, int32_t *accept_len, int32_t *path,
                                int32_t *out_tokens, int32_t *flags)
{
    if (B < 0 || n <= 0 || V <= 0 || max_depth < 0 || !(temperature > 0.0f)) return 1;
    if (parents[0] != -1) return 2;
    for (int32_t i = 1; i < n; ++i) if (parents[i] < -1 || parents[i] >= i) return 2;
    const double tau = (double)temperature;
    int32_t status = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t b = 0; b < B; ++b) {
        const float *tb = target + (int64_t)b * n * V;
        const float *db = draft + (int64_t)b * n * V;
        const int32_t *tk = tokens + (int64_t)b * n;
        int32_t *pb = path + (int64_t)b * (max_depth + 1);
        int32_t *ob = out_tokens + (int64_t)b * (max_depth + 1);
        const uint64_t stream = stream_ids ? stream_ids[b] : (uint64_t)b;
        double *R = (double *)malloc(sizeof(double) * (size_t)V);
        double *q = (double *)malloc(sizeof(double) * (size_t)V);
        for (int32_t d = 0; d <= max_depth; ++d) { pb[d] = -1; ob[d] = -1; }
        int32_t fl = 0, v = 0, d = 0;
        pb[0] = 0;
        for (;;) {
            softmax_row(tb + (int64_t)v * V, V, tau, R);
            softmax_row(db + (int64_t)v * V, V, tau, q);
            int32_t accepted = -1, tries = 0;
            for (int32_t c = v + 1; c < n; ++c) {
                if (parents[c] != v) continue;
                const int32_t s = tk[c];
                const double u = orc_uniform(seed, ((uint64_t)d << 16) | (uint64_t)tries, step, stream, ORC_TAG_RRS);
                if (q[s] > 0.0 && fabs(u - R[s] / q[s]) < ORC_NEAR_RATIO) fl |= 1;
                if (u * q[s] < R[s]) { accepted = c; break; }
                double z = 0.0;
                for (int32_t x = 0; x < V; ++x) z += fmax(0.0, R[x] - q[x]);
                if (z > 0.0)
                    for (int32_t x = 0; x < V; ++x) R[x] = fmax(0.0, R[x] - q[x]) / z;
                if (without_replacement) {
                    q[s] = 0.0;
                    double zq = 0.0;
                    for (int32_t x = 0; x < V; ++x) zq += q[x];
                    if (zq > 0.0) for (int32_t x = 0; x < V; ++x) q[x] /= zq;
                }
                ++tries;
            }
            if (accepted < 0) {
                int32_t near = 0;
                const double u = orc_uniform(seed, ((uint64_t)d << 16) | 0xffffULL, step, stream, ORC_TAG_RRS);
                ob[d] = inverse_cdf(R, V, u, &near);
                if (near) fl |= 2;
                break;
            }
            ob[d] = tk[accepted];
            if (d + 1 > max_depth) {
#pragma omp atomic write
                status = 3;
                break;
            }
            v = accepted;
            ++d;
            pb[d] = v;
        }
        accept_len[b] = d;
        if (flags) flags[b] = fl;
        free(R);
        free(q);
    }
    return status;
}

/* ------------------------------------------------------------------------- */
/* Truncated sampling distributions.  "Speculative decoding" (Zero to        */
/* Frontier), section "When the target samples, keep a guess with           */
/* probability p over q": p and q are the distributions each model really   */
/* samples from, after temperature and truncation such as top-p; the box     */
/* "The speculative sampling rule", special case "A processed target"; box   */
/* "Four ways to lose exactness without noticing": the q of the ratio must   */
/* be the draft's own truncated distribution.                                */
/*   Row r of logits l: tokens in the order (l descending, token id          */
/*   ascending).  top-k keeps the first k (k <= 0 or k >= V: all); then      */
/*   top-p keeps the shortest prefix of those whose mass under               */
/*   softmax(l / T), renormalized over them, reaches top_p (top_p >= 1: all; */
/*   at least one token).  out = l on kept tokens, -inf elsewhere, so that   */
/*   softmax(out / T) is the truncated, renormalized distribution.           */
/*   kept[r] = tokens kept; flags[r] bit0: the top-p prefix mass at the       */
/*   chosen boundary lay within 1e-10 of the target, relative to the set's   */
/*   mass: there weights rounded otherwise (fp64 to ~1e-14 each, summed in    */
/*   another order) could move the boundary by one token.                    */
/*   Per-row k and top_p (top_k_rows, top_p_rows) override the scalars.      */
/* ------------------------------------------------------------------------- */
#define ORC_NEAR_NUCLEUS 1e-10

typedef struct {
    float l;
    int32_t id;
} orc_tok;

static int orc_tok_cmp(const void *a, const void *b)
{
    const orc_tok *x = (const orc_tok *)a, *y = (const orc_tok *)b;
    if (x->l > y->l) return -1;
    if (x->l < y->l) return 1;
    return (x->id > y->id) - (x->id < y->id);
}

ORC_EXPORT int32_t orc_truncate(int32_t R, int32_t V, float temperature, int32_t top_k, float top_p,
                                const int32_t *top_k_rows, const float *top_p_rows, const float *logits, float *out,
                                int32_t *kept, int32_t *flags)
{
    if (R < 0 || V <= 0) return 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t r = 0; r < R; ++r) {
        const float *l = logits + (int64_t)r * V;
        float *o = out + (int64_t)r * V;
        const int32_t k = top_k_rows ? top_k_rows[r] : top_k;
        const double pp = (double)(top_p_rows ? top_p_rows[r] : top_p);
        orc_tok *t = (orc_tok *)malloc(sizeof(orc_tok) * (size_t)V);
        for (int32_t x = 0; x < V; ++x) t[x] = (orc_tok){l[x], x};
        qsort(t, (size_t)V, sizeof(orc_tok), orc_tok_cmp);
        int32_t n = (k > 0 && k < V) ? k : V;
        int32_t fl = 0;
        if (pp < 1.0) {
            const double T = (double)temperature, M = (double)t[0].l;
            double z = 0.0;
            for (int32_t i = 0; i < n; ++i) z += exp(((double)t[i].l - M) / T);
            const double target = pp * z;
            double c = 0.0;
            int32_t m = 0;
            while (m < n) {
                const double before = c;
                c += exp(((double)t[m].l - M) / T);
                ++m;
                if (c >= target) {
                    /* the cut could move by one token: later if c barely reaches the target,
                     * earlier if the prefix before it barely misses (never below one token) */
                    if (fabs(c - target) < ORC_NEAR_NUCLEUS * z ||
                        (m > 1 && fabs(before - target) < ORC_NEAR_NUCLEUS * z))
                        fl |= 1;
                    break;
                }
            }
            n = m > 0 ? m : 1;
        }
        for (int32_t x = 0; x < V; ++x) o[x] = -INFINITY;
        for (int32_t i = 0; i < n; ++i) o[t[i].id] = t[i].l;
        if (kept) kept[r] = n;
        if (flags) flags[r] = fl;
        free(t);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Penalties on the logits, with the drafted prefix as context ([TB]        */
/* section "When the target samples, keep a guess with probability p over   */
/* q": p and q are after temperature, truncation and penalties; box "The    */
/* speculative sampling rule", case "A processed target": they are applied  */
/* with the drafted prefix as context).  The pages name penalties without   */
/* defining them; the usual three are taken:                                */
/*   Row i of sequence b (logits l, [B][n_rows][V]) has the context C =     */
/*   history[b][0 .. hist_len[b]) followed by drafts[b][0 .. min(i,         */
/*   n_drafts)) (drafts NULL: none).  Entries outside [0, V) are skipped,   */
/*   hist_len is clamped into [0, hist_stride].  For every token t with     */
/*   c = (occurrences of t in C) > 0, in fp64 and rounded once to fp32:     */
/*     r = l_t > 0 ? l_t / theta : l_t * theta     (repetition, theta)      */
/*     l_t <- (r - c * freq) - pres                 (frequency, presence)   */
/*   Other tokens keep their logit.  out may be logits itself.              */
/* ------------------------------------------------------------------------- */
ORC_EXPORT int32_t orc_penalize(int32_t B, int32_t n_rows, int32_t V, const float *logits, float *out,
                                const int32_t *history, const int32_t *hist_len, int32_t hist_stride,
                                const int32_t *drafts, int32_t n_drafts, float repetition, float frequency,
                                float presence)
{
    if (B < 0 || n_rows < 0 || V <= 0 || hist_stride < 0 || n_drafts < 0) return 1;
    const double theta = (double)repetition, fr = (double)frequency, pr = (double)presence;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t row = 0; row < (int64_t)B * n_rows; ++row) {
        const int32_t b = (int32_t)(row / n_rows), i = (int32_t)(row % n_rows);
        const float *l = logits + row * V;
        float *o = out + row * V;
        int32_t *count = (int32_t *)calloc((size_t)V, sizeof(int32_t));
        int32_t h = hist_len ? hist_len[b] : 0;
        h = h < 0 ? 0 : (h > hist_stride ? hist_stride : h);
        for (int32_t j = 0; j < h; ++j) {
            const int32_t t = history[(int64_t)b * hist_stride + j];
            if (t >= 0 && t < V) count[t] += 1;
        }
        const int32_t nd = drafts ? (i < n_drafts ? i : n_drafts) : 0;
        for (int32_t j = 0; j < nd; ++j) {
            const int32_t t = drafts[(int64_t)b * n_drafts + j];
            if (t >= 0 && t < V) count[t] += 1;
        }
        for (int32_t t = 0; t < V; ++t) {
            if (count[t] == 0) {
                o[t] = l[t];
                continue;
            }
            const double x = (double)l[t];
            const double r = x > 0.0 ? x / theta : x * theta;
            const double cf = (double)count[t] * fr;
            o[t] = (float)((r - cf) - pr);
        }
        free(count);
    }
    return 0;
}
