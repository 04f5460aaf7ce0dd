/*
 * specverify.h -- C ABI of libspecverify, the verify step of speculative decoding
 * on one AMD Instinct MI355X (gfx950).
 *
 * The verify step (sources cited by page title and section):
 *   - "Speculative decoding" (Zero to Frontier textbook, ch. 20, section 20.5), below [TB];
 *   - "Speculative-Decoding" (s1mplewind blog, Medusa notes), below [MED];
 *   - "Speculative Decoding: The Art of Guessing Well" (astralord blog), below [AG].
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is DEVICE memory owned by the caller, unless marked "host".
 *     Descriptors are read on the host during the call and not kept.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the null stream)
 *     and never synchronizes the host.
 *   - Argument checks run on the host before any launch and return SV_ERR_INVALID_ARG,
 *     SV_ERR_UNSUPPORTED or SV_ERR_WORKSPACE without touching the device.  Errors that
 *     only the data can show (a bad parent, a token id out of range) are written to the
 *     device status words the calls document.  A failed launch returns SV_ERR_HIP.
 *   - Workspaces: `*_workspace()` returns the byte size a call needs for a descriptor
 *     (0 for a call that needs none, or for a descriptor the call would reject).  The
 *     caller allocates it (device memory, 256-byte aligned).  Its first 128 KiB hold the
 *     call's completion counters: they must be zero when the workspace is first used, and
 *     every call leaves them zero again (partial results live after them).  So one
 *     workspace, zero-filled once, may serve any sequence of calls of any entry point and
 *     shape, provided the calls do not overlap in time (e.g. they share one stream).
 *   - The library allocates no memory and keeps no state between calls: whatever a call
 *     needs (device attributes, occupancy) it asks the runtime for during the call.  The
 *     one exception is sv_spec_accept_static's fixed device array and the per-device
 *     record of its address.
 *     Completion counters return to zero at the end of every kernel that uses them, and
 *     a launch that fails never runs, so a call that returns SV_ERR_HIP leaves its
 *     workspace's counter region zero as well.
 *   - No C++ exception crosses this interface.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define SV_API __attribute__((visibility("default")))
#else
#define SV_API
#endif

typedef enum sv_status {
    SV_OK = 0,
    SV_ERR_INVALID_ARG = 1,  /* a null pointer, a negative size, inconsistent shapes      */
    SV_ERR_UNSUPPORTED = 2,  /* a valid request the library does not implement (e.g. D=96) */
    SV_ERR_WORKSPACE = 3,    /* workspace pointer null or smaller than *_workspace()     */
    SV_ERR_HIP = 4           /* a HIP launch failed                                       */
} sv_status;

typedef enum sv_dtype { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

/* GREEDY: argmax decisions on raw logits.  SAMPLE: temperature softmax and speculative
 * sampling; SAMPLE with temperature == 0 is GREEDY ([TB] "When the target samples...":
 * as the temperature goes to 0 both models approach their argmax).                      */
typedef enum sv_mode { SV_GREEDY = 0, SV_SAMPLE = 1 } sv_mode;

/* Verification rule of sv_spec_accept in SAMPLE mode (GREEDY mode is greedy matching   */
/* under every rule: each reduces to it when both models are one-hot).                    */
/*   TOKEN:  speculative sampling, token by token ([TB] "The speculative sampling rule").  */
/*   BLOCK:  block verification ([AG] "Block verification"): the drafted prefix is kept    */
/*           jointly, by running weights w_k = min(1, w_{k-1} p_k(x_k)/q_k(x_k)).          */
/*   GUMBEL: Gumbel-coupled verification ([AG] "Sampling with shared noise"): the target    */
/*           samples every position by Gumbel-max with noise it shares with the drafter,  */
/*           and the longest prefix where the drafts equal those samples is kept.          */
typedef enum sv_rule { SV_RULE_TOKEN = 0, SV_RULE_BLOCK = 1, SV_RULE_GUMBEL = 2 } sv_rule;

/* CAUSAL: bottom-right-aligned causal mask of a chain ([TB] "Checking several tokens costs
 * about as much as writing one").  TREE: ancestor-or-self mask of a token tree ([TB] box
 * "Token tree and tree attention"; [MED] "Attention Tree").                              */
typedef enum sv_mask { SV_MASK_CAUSAL = 0, SV_MASK_TREE = 1 } sv_mask;

/* Counter-based uniforms: Philox4x64-10 (Salmon et al., SC'11) with key (seed, 0) and
 * counter (index, step, stream, tag); u = (2*(w0 >> 12) + 1) * 2^-53, exact in fp64 and
 * inside (0,1).  The pages ask for independent uniforms and name no generator.
 * stream_ids: device [B] uint64 stream of each sequence, or NULL for stream = b.          */
typedef struct sv_philox {
    uint64_t seed;
    uint64_t step;
    const uint64_t *stream_ids;
} sv_philox;

/* ---------------------------------------------------------------------------------- */
/* sv_build_tree_mask -- [TB] box "Token tree and tree attention" and exercise "The tree */
/* attention mask".  A tree of n nodes is a parent array, par(i) in {-1, 0, ..., i-1}    */
/* (parents listed before children; -1 follows the last committed token; several -1     */
/* entries make a forest).  Node i may attend to every prefix position and to node j     */
/* exactly when j == i or j is an ancestor of i; its position id is prefix_len + depth(i),*/
/* depth = number of ancestors.                                                          */
/*   parents    device int32 [n]                                                         */
/*   bits       device uint32 [n][ceil(n/32)]: bit (j % 32) of word j / 32 of row i is    */
/*              set iff node i sees node j (the node-to-node block; the prefix block is  */
/*              all ones and is not stored).  This is the tree_bits layout of            */
/*              sv_verify_attention.                                                     */
/*   depth      device int32 [n];  pos  device int64 [n] = prefix_len + depth            */
/*   dev_status device int32 [1]: 0 when every parent is valid, else 1 + the first node   */
/*              whose parent is not in [-1, i).  Rows of such trees are unspecified.     */
/* Errors: n < 1 or prefix_len < 0 or a null pointer -> SV_ERR_INVALID_ARG.              */
/* ---------------------------------------------------------------------------------- */
SV_API sv_status sv_build_tree_mask(const int32_t *parents, int32_t n, int32_t prefix_len,
                             uint32_t *bits, int32_t *depth, int64_t *pos,
                             int32_t *dev_status, void *stream);

/* ---------------------------------------------------------------------------------- */
/* sv_verify_attention -- the multi-token attention of a verification pass.             */
/* [TB] "Checking several tokens costs about as much as writing one": each new token     */
/* attends to the whole cache and to the new tokens before it; [TB] box "Token tree and  */
/* tree attention" for trees; query head h reads KV head h / (Hq / Hkv).                 */
/* For sequence b with P = prefix_len[b], row i in [0, n_q) of query head h computes     */
/*   s_t = scale * <q[b][i][h], k_t>,  t visible;  o = sum_t softmax(s)_t v_t            */
/* over t in [0, P) plus t = P + j for new token j visible from i: j <= i (CAUSAL) or    */
/* bit j of tree row i (TREE).  lse = log sum_t exp(s_t) (natural log).                  */
/* Layout (element strides; the D elements of a row are contiguous):                     */
/*   q    [B][n_q][Hq][D] at q + b*q_sb + i*q_st + h*q_sh                                */
/*   k, v cache of sequence b starts at element kv_off[b] (device int64 [B]); token t of */
/*        KV head g is at kv_off[b] + g*kv_sh + t*kv_st.  The cache must hold P + n_q     */
/*        tokens: the keys/values of the n_q new tokens are written before this call.    */
/*        kv_off may be NULL (a dense cache): sequence b then starts at element b*kv_sb,  */
/*        and every sequence must own max_prefix + n_q token slots, since the kernel may */
/*        read any of them (rows past P + n_q are read but never used).                  */
/*   prefix_len  device int32 [B];  max_prefix (host) must bound every prefix_len[b]:    */
/*        it sizes the launch; a sequence whose P exceeds it, or is negative, reads       */
/*        nothing and gets NaN output rows (and NaN lse).                                */
/*   tree_bits   TREE only: device uint32 rows as produced by sv_build_tree_mask, for    */
/*        n_q nodes; sequence b uses tree_bits + b*tree_sb (tree_sb = 0: one shared tree).*/
/*   out  [B][n_q][Hq][D] of `dtype` at out + b*o_sb + i*o_st + h*o_sh                   */
/*   lse  optional fp32 [B][n_q][Hq] contiguous, or NULL                                 */
/* dtype: SV_BF16 (bf16 in and out, fp32 accumulation, MFMA; key splits hand their       */
/*        partial outputs to the merge as o / sum rounded to bf16 -- a convex combination  */
/*        of V rows, so at most one more bf16 rounding of the output) or SV_F32 (fp32     */
/*        throughout).                                                                   */
/* scale > 0 (else SV_ERR_INVALID_ARG).                                                  */
/* split_keys: keys per work split (a tuning knob, rounded up to the kernel's tile        */
/*        granularity); 0 picks a split that fills the GPU.                              */
/* Supported: D in {64, 128}; Hq % Hkv == 0; n_q >= 1.  bf16 also needs 16-byte aligned  */
/* q, k, v, strides, kv_sb and kv_off[b] that are multiples of 8 elements, and out and  */
/* its strides aligned to 4 elements (else SV_ERR_UNSUPPORTED; kv_off is not checked).   */
/* bf16 calls with at most 32 query rows per KV head (n_q x Hq/Hkv) take B <= 65535.     */
/* Measurement events (optional, hipEvent_t, NULL when unused; no result depends on them):*/
/*   ev_kernel_start / ev_kernel_stop: the bf16 main attention kernel is launched so that  */
/*        they take its own start and end times (the span a kernel trace reports,         */
/*        without the dispatch ahead of it);                                            */
/*   ev_call_stop: the end time of the call's last kernel -- the split combine's own end  */
/*        when the call has one (launched the same way), else the main kernel's end.      */
/*        ev_kernel_start to ev_call_stop spans the whole attention pass on the GPU.      */
/* ---------------------------------------------------------------------------------- */
typedef struct sv_attn_desc {
    sv_dtype dtype;
    sv_mask mask;
    int32_t B, n_q, Hq, Hkv, D;
    int32_t max_prefix;
    int32_t split_keys;
    float scale;
    const void *q;
    int64_t q_sb, q_st, q_sh;
    const void *k;
    const void *v;
    const int64_t *kv_off;
    int64_t kv_sh, kv_st;
    int64_t kv_sb;
    const int32_t *prefix_len;
    const uint32_t *tree_bits;
    int64_t tree_sb;
    void *out;
    int64_t o_sb, o_st, o_sh;
    float *lse;
    void *ev_kernel_start;
    void *ev_kernel_stop;
    void *ev_call_stop;
} sv_attn_desc;

SV_API size_t sv_verify_attention_workspace(const sv_attn_desc *desc);
SV_API sv_status sv_verify_attention(const sv_attn_desc *desc, void *workspace, size_t workspace_bytes,
                              void *stream);

/* ---------------------------------------------------------------------------------- */
/* sv_spec_accept -- acceptance of one round for B sequences of gamma drafts each.       */
/* GREEDY: [TB] box "A round of greedy speculative decoding": z_i = argmax of target row */
/*   i (raw fp32 logits, ties -> lowest id); J = number of leading drafts with x_i = z_i;*/
/*   emit x_0..x_{J-1} then z_J.  Draft logits are not read (may be NULL).               */
/* SAMPLE: [TB] boxes "The speculative sampling rule" and "A round of speculative        */
/*   sampling"; [AG] "Speculative sampling".  p_i = softmax(target_i / T),               */
/*   q_i = softmax(draft_i / T) (the same temperature on both models);                   */
/*   for i = 0..gamma-1 accept x_i iff u_i * q_i(x_i) < p_i(x_i), u_i the Philox uniform */
/*   (index i, tag 0x53560001), stopping at the first rejection; J = number accepted.    */
/*   The extra token is an inverse-CDF draw in token-id order, with the uniform of index */
/*   gamma, from r = max(0, p_J - q_J) when J < gamma, else from p_gamma ([TB] section   */
/*   "Speculative verification in PyTorch": a zero draft row after the last draft).      */
/*   A residual with zero mass falls back to p_J.                                        */
/* Precision: exponentials in fp32, sums and the CDF in fp64; a decision can differ from */
/* exact arithmetic only when its uniform lies within about 1e-6 of its threshold.       */
/*   target_logits device fp32 [B][gamma+1][V]; draft_logits fp32 [B][gamma][V] (SAMPLE)*/
/*   draft_tokens  device int32 [B][gamma], each in [0, V)                               */
/*   accept_len    device int32 [B] = J                                                  */
/*   out_tokens    device int32 [B][gamma+1]: J accepted drafts, the extra token, then -1*/
/*   alpha         optional device fp32 [B][gamma]: sum_x min(p_i, q_i) ([TB] "The       */
/*                 speculative sampling rule"); SAMPLE only (NaN under GREEDY); NULL     */
/*                 skips its extra pass over the rows                                    */
/*   dev_status    optional device int32 [B]: 0, or 2 when a draft token is outside      */
/*                 [0, V) (that sequence's outputs are then unspecified)                 */
/*   rule          SV_RULE_TOKEN (the above), SV_RULE_BLOCK or SV_RULE_GUMBEL (SAMPLE     */
/*                 mode; see below).  The workspace size depends on it.                   */
/* BLOCK ([AG] "Block verification"): with p_k, q_k the target rows and draft rows of     */
/*   position k (row k-1) and w_0 = 1, w_k = min(1, w_{k-1} p_k(x_k)/q_k(x_k)) (a drafted  */
/*   token with q = 0 gives 1 if p > 0, else 0), prefix k survives when its uniform       */
/*   (index k-1) is <= h_k = m_k / (m_k + 1 - w_k) (1 when w_k = 1), m_k =                 */
/*   sum_x (w_k p_{k+1}(x) - q_{k+1}(x))+ and m_gamma = w_gamma; J = the longest surviving */
/*   prefix, and the extra token is an inverse-CDF draw (index gamma) from                */
/*   (w_J p_{J+1} - q_{J+1})+ (q_{gamma+1} = 0; a zero residual falls back to p_{J+1}).    */
/* GUMBEL ([AG] "Sampling with shared noise"): y_i = argmax_x (l_i(x)/T + g_i(x)),         */
/*   g = -log(-log u), u of token x at position i the word x mod 4 of the Philox block    */
/*   with counter (x div 4, step, stream, 0x53560003 + 2^32 i); J = the first i < gamma    */
/*   with x_i != y_i (else gamma); emits x_0..x_{J-1}, y_J.  Draft logits are not read    */
/*   (the drafter used the same noise); scores in fp64, ties to the lowest token.          */
/* RAGGED LENGTHS ([TB] section "Choosing how much to verify at every step": a step      */
/*   verifies its own number of drafts per request):                                     */
/*   draft_len     optional device int32 [B]; sequence b verifies only its first          */
/*                 L_b = draft_len[b] drafts, 0 <= L_b <= gamma.  Its results are exactly  */
/*                 those of the same call with gamma = L_b on its first L_b + 1 target     */
/*                 rows, L_b draft rows and tokens (so the extra token takes the uniform   */
/*                 of index L_b, and L_b = 0 is one draw from target row 0); rows past     */
/*                 them are neither read nor needed.  accept_len <= L_b; out_tokens as     */
/*                 above, then -1 to gamma + 1 entries; alpha NaN past L_b.  NULL: every   */
/*                 sequence verifies gamma drafts.  The layouts keep their gamma strides.  */
/*                 The result is exact only when L_b does not depend on the drafted tokens  */
/*                 themselves (the section's warning box "Trimming a draft can break       */
/*                 exactness"): the caller's choice, which the library cannot check.        */
/*   dev_status    3 when draft_len[b] is outside [0, gamma] (the sequence is then taken   */
/*                 with L_b clamped into it; its outputs are unspecified)                  */
/* Supported: 1 <= gamma <= 64, 1 <= V, B <= 32768.                                      */
/* ---------------------------------------------------------------------------------- */
typedef struct sv_accept_desc {
    sv_mode mode;
    int32_t B, gamma, V;
    float temperature;
    const float *target_logits;
    const float *draft_logits;
    const int32_t *draft_tokens;
    sv_philox rng;
    int32_t *accept_len;
    int32_t *out_tokens;
    float *alpha;
    int32_t *dev_status;
    sv_rule rule;
    const int32_t *draft_len;
} sv_accept_desc;

SV_API size_t sv_spec_accept_workspace(const sv_accept_desc *desc);
SV_API sv_status sv_spec_accept(const sv_accept_desc *desc, void *workspace, size_t workspace_bytes,
                         void *stream);

/* ---------------------------------------------------------------------------------- */
/* sv_spec_accept_static -- sv_spec_accept for callers that cannot allocate device       */
/* memory (code under HIP graph capture, tight serving loops, harnesses that forbid      */
/* allocation): the same kernels and results, with the workspace taken from a fixed      */
/* device array inside the library of SV_STATIC_SCRATCH_BYTES per GPU (held from the      */
/* first call on that GPU until the process ends; its address is looked up on that first */
/* call, which should therefore not itself be under graph capture).  The calling thread's*/
/* current device must be the stream's.  Inputs and outputs as in sv_spec_accept.        */
/* Errors: as sv_spec_accept; SV_ERR_WORKSPACE when sv_spec_accept_workspace(desc)       */
/* exceeds SV_STATIC_SCRATCH_BYTES (checked on the host before anything else).  Every    */
/* call on one GPU shares the array: calls that overlap in time on one GPU race (issue   */
/* them on one stream, or order them).  The call allocates nothing.                      */
/* ---------------------------------------------------------------------------------- */
#define SV_STATIC_SCRATCH_BYTES (16u << 20)
SV_API sv_status sv_spec_accept_static(const sv_accept_desc *desc, void *stream);

/* ---------------------------------------------------------------------------------- */
/* sv_tree_walk -- verification of a token tree by a walk from the root.                 */
/* GREEDY: [TB] section "Token trees check several guesses at once": start at the root,  */
/*   move to the child equal to the target's choice, repeat, and at the first node with  */
/*   no such child emit the target's choice.  SAMPLE: [MED] section "Attention Tree":    */
/*   sample from the target at the node, look for that token among its children, and go  */
/*   down level by level until no child matches.                                         */
/* Node 0 is the root (the last committed token, parent -1); row v of the logits is the  */
/* target's next-token distribution after node v.  At depth d the choice at node v is    */
/* argmax(logits[v]) (GREEDY) or an inverse-CDF draw from softmax(logits[v] / T) with    */
/* the Philox uniform (index d, tag 0x53560002) (SAMPLE); the walk moves to the first    */
/* child of v in node order whose token equals it.                                       */
/*   logits   device fp32 [B][n][V];  tokens device int32 [B][n];                        */
/*   parents  device int32 [n], shared by the batch (parents[0] == -1, parents[i] < i)   */
/*   max_depth (host): the depth of the deepest node (capacity of path and out_tokens)   */
/*   accept_len device int32 [B] = J (accepted nodes)                                    */
/*   path       device int32 [B][max_depth+1] = (0, n_1, ..., n_J, -1, ...)              */
/*   out_tokens device int32 [B][max_depth+1] = (tokens of n_1..n_J, the choice at n_J,  */
/*              -1, ...)                                                                 */
/*   dev_status optional device int32 [B]: 0, 5 (RRS, see below), or 3 when the walk    */
/*              would go below                                                           */
/*              max_depth: it then stops at its node at depth max_depth and emits the    */
/*              choice there as the extra token (accept_len = max_depth; still a draw    */
/*              from the target at that node)                                            */
/*   rule       SV_WALK_MATCH: the walk above.  SAMPLE mode only (GREEDY is the greedy     */
/*              walk under every rule): SV_WALK_RRS, recursive rejection ([TB] box         */
/*              "Recursive rejection at a node with several children"): the children      */
/*              s_1..s_k of node v (node order) were drawn i.i.d. from the drafter's q_v   */
/*              = softmax(draft_logits[v] / T); with R_1 = p_v, child i is accepted when   */
/*              u q(s_i) < R_i(s_i), R_{i+1} = (R_i - q)+ normalized, and if every child   */
/*              is rejected (or v is a leaf) the extra token is drawn from R_{k+1};        */
/*              SV_WALK_RRS_WOR, the same for children drawn without replacement (same    */
/*              section): a rejected token is also removed from q, which is renormalized. */
/*              Uniforms: tag 0x53560004, index 2^16 d + i for try i at depth d, 2^16 d +  */
/*              0xffff for the draw.  An accepted child at max_depth is emitted as the    */
/*              extra token (status 3).                                                   */
/*   draft_logits  RRS: device fp32 [B][n][V], row v = the drafter's logits at node v       */
/*   max_children  RRS: a bound on the children of any node (1..64; it sets the number of  */
/*              passes per level); a node with more sets status 5 and ends its walk       */
/* Supported: 1 <= n, 0 <= max_depth <= 63, 1 <= V, B <= 32768.                          */
/* ---------------------------------------------------------------------------------- */
typedef enum sv_walk_rule { SV_WALK_MATCH = 0, SV_WALK_RRS = 1, SV_WALK_RRS_WOR = 2 } sv_walk_rule;

typedef struct sv_walk_desc {
    sv_mode mode;
    int32_t B, n, V, max_depth;
    float temperature;
    const float *logits;
    const int32_t *tokens;
    const int32_t *parents;
    sv_philox rng;
    int32_t *accept_len;
    int32_t *path;
    int32_t *out_tokens;
    int32_t *dev_status;
    sv_walk_rule rule;
    const float *draft_logits;
    int32_t max_children;
} sv_walk_desc;

SV_API size_t sv_tree_walk_workspace(const sv_walk_desc *desc);
SV_API sv_status sv_tree_walk(const sv_walk_desc *desc, void *workspace, size_t workspace_bytes,
                       void *stream);

/* ---------------------------------------------------------------------------------- */
/* sv_kv_commit -- the KV-cache commit after a round.  [TB] section "Keeping the caches   */
/* consistent after a rejection": after J acceptances the entries of the accepted drafts */
/* are kept and the rejected ones discarded; the correction or bonus token has no entry  */
/* yet.  A chain rolls back by moving its length; a tree also gathers the accepted       */
/* branch's entries, scattered among discarded siblings, into consecutive slots ([AG]    */
/* "Verification bottlenecks": KV cache bookkeeping).                                    */
/* The verification pass wrote node (or chain row) j of sequence b at position P_b + j,  */
/* node 0 being the last committed token.  Afterwards position P_b + k holds the entry of */
/* path node k (k = 1..J_b) and new_len[b] = P_b + 1 + J_b.                              */
/*   k, v       the caches, layout as sv_verify_attention (kv_off or dense kv_sb; token t */
/*              of KV head g at kv_off[b] + g*kv_sh + t*kv_st, D contiguous elements of   */
/*              `dtype`); rows are moved in place                                        */
/*   prefix_len device int32 [B]: P_b;  accept_len device int32 [B]: J_b (from           */
/*              sv_spec_accept or sv_tree_walk)                                           */
/*   path       device int32 [B][path_stride]: sv_tree_walk's path (node 0 first), or    */
/*              NULL for chains (only the length moves)                                  */
/*   new_len    device int32 [B]: P_b + 1 + J_b; may be prefix_len itself (in place)     */
/*   dev_status optional device int32 [B]: 0, or 4 when J_b is outside [0, n_q) or a     */
/*              path node k is outside [k, n_q) (that sequence is left untouched)         */
/* Supported: path_stride <= 65 (a walk's max_depth <= 63); D * element size and the     */
/* strides multiples of 16 bytes, k and v 16-byte aligned (else SV_ERR_UNSUPPORTED).      */
/* ---------------------------------------------------------------------------------- */
typedef struct sv_commit_desc {
    sv_dtype dtype;
    int32_t B, n_q, Hkv, D;
    void *k;
    void *v;
    const int64_t *kv_off;
    int64_t kv_sb, kv_sh, kv_st;
    const int32_t *prefix_len;
    const int32_t *accept_len;
    const int32_t *path;
    int32_t path_stride;
    int32_t *new_len;
    int32_t *dev_status;
} sv_commit_desc;

SV_API sv_status sv_kv_commit(const sv_commit_desc *desc, void *stream);

/* ---------------------------------------------------------------------------------- */
/* sv_truncate -- top-k and top-p (nucleus) truncation of logit rows, the processing     */
/* that makes p and q the distributions the two models really sample from ([TB] section  */
/* "When the target samples, keep a guess with probability p over q", and box "The       */
/* speculative sampling rule", case "A processed target": temperature and top-p are     */
/* applied to the target with the drafted prefix as context).  The draft's rows must go  */
/* through the same processing before they enter the ratio: the box "Four ways to lose   */
/* exactness without noticing" names the draft's logits before its top-p cut as a wrong */
/* q.  Feed the output rows to sv_spec_accept (or sv_tree_walk) with the same T.          */
/* Tokens of a row are ordered by logit, highest first, equal logits by token id, lowest */
/* first.  top-k keeps the first k of them (off when k <= 0 or k >= V).  top-p then keeps  */
/* the shortest prefix of what top-k kept whose mass under softmax(l / T), taken over    */
/* that kept set, reaches top_p times the set's total mass, and never fewer than one     */
/* token (off when top_p >= 1 or NaN; top_p <= 0 keeps one token).  A row whose logits    */
/* are all -inf is left as it is by top-p.                                                 */
/*   logits      device fp32 [R][V]                                                        */
/*   out         device fp32 [R][V]: the logit of each kept token, -inf elsewhere; may be */
/*               `logits` itself (in place)                                                */
/*   kept        optional device int32 [R]: the number of kept tokens of each row          */
/*   top_k_rows  optional device int32 [R]: per-row k, replaces top_k                     */
/*   top_p_rows  optional device fp32 [R]: per-row top_p, replaces top_p                  */
/*   temperature T > 0 and finite (weights of top-p; read even when top-p is off)         */
/* Top-p weights are 2^((l - max) log2(e) / T) in fp64 (to about 2e-14 relative), summed */
/* exactly as integers in units of 2^-62 of the largest one, so the kept set does not     */
/* depend on the order of the sums, and it can differ from the exact one only where the  */
/* cut lies within about 1e-13 of the set's mass, relative.  NaN or +inf logits: results */
/* unspecified.                                                                           */
/* Workspace (optional): with at least sv_truncate_workspace(desc) bytes (nonzero only for */
/* R up to a quarter of the compute units and V >= 16384), the first level and, when it   */
/* leaves few tokens, the gathering of every row are spread over many workgroups: for a    */
/* few rows about twice as fast; the result is the same.  With less (or NULL) the call    */
/* runs without it.  Shared like the other calls' workspaces.                              */
/* Errors: R < 0, V < 1, T not in (0, inf), NaN top_p, or (R > 0) a null logits or out  */
/*   -> SV_ERR_INVALID_ARG.  R == 0 launches nothing.  out and logits are the same rows or */
/*   do not overlap.                                                                        */
/* Supported: 1 <= V <= 2^24 (else SV_ERR_UNSUPPORTED), R <= 2^31 - 1.                    */
/* ---------------------------------------------------------------------------------- */
typedef struct sv_trunc_desc {
    int32_t R, V;
    float temperature;
    int32_t top_k;
    float top_p;
    const int32_t *top_k_rows;
    const float *top_p_rows;
    const float *logits;
    float *out;
    int32_t *kept;
} sv_trunc_desc;

SV_API size_t sv_truncate_workspace(const sv_trunc_desc *desc);
SV_API sv_status sv_truncate(const sv_trunc_desc *desc, void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------- */
/* sv_penalize -- repetition, frequency and presence penalties on logit rows, in place,   */
/* with the drafted prefix as context ([TB] section "When the target samples, keep a     */
/* guess with probability p over q": p and q are after temperature, truncation and       */
/* penalties; box "The speculative sampling rule", case "A processed target": they are   */
/* applied with the drafted prefix as context).  The pages do not define the penalties;  */
/* the usual three are taken.  Row i of sequence b has the context C = history[b][0 ..   */
/* hist_len[b]) followed by draft_tokens[b][0 .. min(i, n_drafts)).  For every token t   */
/* seen c > 0 times in C, with l its logit, in fp64 (no fused operations) and rounded    */
/* once to fp32:                                                                          */
/*     r = l > 0 ? l / repetition : l * repetition;   l <- (r - c * frequency) - presence  */
/* Other logits are not touched.  Use it on the target rows (n_rows = gamma + 1) and the  */
/* draft rows (n_rows = gamma) with the same drafts, before temperature and sv_truncate. */
/*   logits       device fp32 [B][n_rows][V], penalized in place                         */
/*   history      optional device int32 [B][hist_stride]: each sequence's tokens so far  */
/*   hist_len     optional device int32 [B]: valid entries (clamped into [0, hist_stride]);*/
/*                NULL: hist_stride each                                                   */
/*   draft_tokens optional device int32 [B][n_drafts]                                     */
/*   Entries outside [0, V) are skipped.  repetition 1, frequency 0, presence 0: no change. */
/* Work is proportional to the history's distinct tokens times the rows, not to V.  Up to */
/* 8192 history entries per sequence they are counted in LDS; beyond, in a count over the */
/* vocabulary in the workspace (4 V + 4 hist_stride bytes per sequence).  The call reads  */
/* only workspace entries it wrote first, so it shares a workspace with the other entry   */
/* points as they do.                                                                      */
/* Errors: B, n_rows or hist_stride negative, V < 1, repetition not in (0, inf),          */
/*   frequency or presence not finite, or (rows > 0) a null logits -> SV_ERR_INVALID_ARG; */
/*   n_drafts > 64, B > 32768 or more than 65535 chunks of 1024 history entries ->        */
/*   SV_ERR_UNSUPPORTED.  After SV_ERR_HIP zero the workspace again before reusing it.    */
/* ---------------------------------------------------------------------------------- */
typedef struct sv_penalty_desc {
    int32_t B, n_rows, V;
    float *logits;
    const int32_t *history;
    const int32_t *hist_len;
    int32_t hist_stride;
    const int32_t *draft_tokens;
    int32_t n_drafts;
    float repetition, frequency, presence;
} sv_penalty_desc;

SV_API size_t sv_penalize_workspace(const sv_penalty_desc *desc);
SV_API sv_status sv_penalize(const sv_penalty_desc *desc, void *workspace, size_t workspace_bytes, void *stream);

/* Human-readable name of a status code (static storage). */
SV_API const char *sv_status_string(sv_status status);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
