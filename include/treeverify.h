/*
 * treeverify.h -- C ABI of the MI355X (gfx950) draft-tree verify path.
 *
 * One verify round of draft-tree speculative decoding on one GPU:
 *   tree_beam_step, tree_select_candidates, tree_retrieve_links
 *                        the tree from the drafter's candidate pool
 *   tree_build_masks     parents -> depth, 64-bit ancestor masks, positions
 *   tree_attention       paged prefix + masked tree window -> out, base-2 LSE
 *   tree_attention_mla   prefix + window + merge with K and V read from one
 *                        MLA latent row per token
 *   verify_tree_greedy   draft tokens, target argmax -> accepted path
 *   tree_sample_gumbel   logits -> target draws keyed by (seed, position),
 *                        for the sampled verify
 *   verify_tree_rejection  target rows, draft tokens -> accepted path by
 *                        tree rejection sampling
 *   compact_window_rows  accepted path -> rows moved to the window's front
 *   tree_shift_positions load_step / compact_rows position shifts
 *
 * Sources (page title, section):
 *  [DTS] "Draft-tree speculation" (tokenspeed design notes)
 *  [ETA] "EAGLE Tree Attention candidate layout, positions and visibility"
 *        (SGLang EAGLE tree-verify analysis)
 *  [MEM] "Medusa, EAGLE-1/2/3, MTP, and tree attention" (course chapter)
 *  [DDT] "From Greedy to Sampling: The Architecture of Choice in DDTree
 *        Speculative Decoding"
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers owned by the caller, unless marked "host".
 *    Arrays are dense row-major with the shapes given.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues kernels on it: no host synchronisation, no allocation, no
 *    global mutable state, so calls can be captured in a HIP graph.
 *  - All arguments are checked on the host before anything is launched; a
 *    violation returns a non-zero status, launches nothing, and
 *    tav_last_error() names every failed check ([DTS] "Scope": refuse up
 *    front and report every blocker together).  Device-side data that the
 *    host cannot see (parent arrays, page-table entries, per-request lengths)
 *    never causes an out-of-bounds access; what happens to it is stated per
 *    entry point.
 */
#ifndef TREEVERIFY_H
#define TREEVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TAV_OK = 0,
    TAV_ERR_INVALID_ARG = 1, /* null pointer, negative size, limit violated */
    TAV_ERR_UNSUPPORTED = 2, /* well-formed but outside what is implemented */
    TAV_ERR_WORKSPACE = 3,   /* workspace too small or misaligned          */
    TAV_ERR_HIP = 4          /* a HIP launch failed                         */
} tav_status;

typedef enum {
    TAV_F32 = 0,      /* IEEE fp32 */
    TAV_BF16 = 1,     /* bfloat16 */
    TAV_FP8_E4M3 = 2  /* tree_attention only: K/V caches in FP8 E4M3 (1 byte:
                         sign, 4 exponent bits with bias 7, 3 mantissa bits, no
                         infinities, NaN at all ones; unscaled), q and out bf16 */
} tav_dtype;

/* Text of the last failure on the calling thread ("" after a success). */
const char *tav_last_error(void);

/* Library version string. */
const char *tav_version(void);

/*
 * Ancestor masks, depth and positions of each request's draft tree.
 * [ETA] section 1: row i sees key j of the window iff j == i or j is an
 * ancestor of i; [DTS] "One tree attention ...": that visibility is one
 * 64-bit mask per row (bit j = window node j); [ETA] section 2 and [DTS]
 * "Position follows depth, slot follows node index": node i's RoPE position
 * is vc + depth[i].
 *
 * parents    int32 [B][N]  node 0 is the root (-1); parents[i] in [0, i)
 * B, N       B >= 0, 1 <= N <= 64
 * vc         int32 [B] or NULL (0): committed prefix length per request
 * depth      int32 [B][N]  out: number of ancestors
 * masks      uint64 [B][N] out: bit i and the bits of all ancestors of i
 * positions  int32 [B][N] or NULL: out vc[b] + depth
 * tree_error int32 [B] or NULL: out 0, or 1 + the first node whose parent is
 *            invalid ([MEM] "Building the mask, for real": a missing parent
 *            is rejected, never treated as a root).  For such a request
 *            masks are 0 and depth/positions are -1.
 */
tav_status tree_build_masks(const int32_t *parents, int32_t B, int32_t N,
                            const int32_t *vc, int32_t *depth, uint64_t *masks,
                            int32_t *positions, int32_t *tree_error, void *stream);

/*
 * In-place position shift: positions[b][i] += direction * (depth[b][i] - i).
 * direction +1 is load_step (vc + i -> vc + depth), -1 is compact_rows
 * (vc + depth -> vc + i); the two cancel for any depth buffer ([DTS]
 * "Position follows depth, slot follows node index").
 * positions, depth int32 [B][N]; B >= 0; 1 <= N <= 64; direction = +1 or -1.
 */
tav_status tree_shift_positions(int32_t *positions, const int32_t *depth, int32_t B,
                                int32_t N, int32_t direction, void *stream);

/*
 * Bytes of device workspace tree_attention needs for these sizes (the same
 * arguments it takes).  0 means the arguments are invalid.
 */
size_t tree_attention_workspace_size(tav_dtype dtype, int32_t B, int32_t R, int32_t Hq,
                                     int32_t Hkv, int32_t D, int32_t max_prefix_len,
                                     int32_t prefix_window, int32_t page_size);

/*
 * Tree attention over a paged KV cache: every row attends the committed
 * prefix plus exactly the window nodes its ancestor mask selects, and the
 * result carries the base-2 log-sum-exp of the whole visible set.
 * [DTS] "One tree attention: the leaf's decode for the prefix, a small kernel
 * for the tree" (the cascade: a prefix decode, a masked window part, and a
 * merge of both through their base-2 LSE); [ETA] section 4 (the same cascade
 * on FlashAttention: common prefix, per-query ancestor suffix, LSE merge).
 *
 * Row r of request b, query head h uses kv head h / (Hq / Hkv) and sees, with
 * P = prefix_len[b]:
 *   prefix keys at logical positions [p_lo, P), p_lo = max(0, P -
 *   prefix_window) when prefix_window > 0 (a frozen sliding window, [DTS]
 *   "One tree attention ...", lanes with per-row tables), else 0; and
 *   window node j at logical position P + j for every j < W whose bit is set
 *   in masks[b][r].
 * Scores are sm_scale * q.k (sm_scale <= 0 means 1/sqrt(D)); keys that are
 * not visible are never used, so non-finite values there never reach an
 * output.  A row with no visible key gets out = 0, lse2 = -inf.
 *
 * q          [B][R][Hq][D] dtype, contiguous
 * k_cache, v_cache  paged pools of dtype: element (page, kv head g, slot s,
 *            channel d) at page*stride_page + g*stride_head + s*stride_token + d
 *            (strides in elements; channels contiguous; e.g. HND
 *            [pages][Hkv][page_size][D] or NHD [pages][page_size][Hkv][D]).
 *            Pointers and strides must give 16-byte aligned rows, and
 *            stride_token must be below 2^27 bytes.
 * num_pages  pages in each pool; page-table entries outside [0, num_pages)
 *            are clamped into it (memory-safe, results for that key undefined)
 * page_table int32 [B][max_pages]: logical position t of request b lives in
 *            page page_table[b][t / page_size] at slot t % page_size
 * page_size  a power of two in [1, 1024]
 * prefix_len int32 [B]: P per request, in [0, max_prefix_len] (values
 *            outside are clamped); the window keys follow it
 * max_prefix_len  host bound on prefix_len; max_pages * page_size must be
 *            >= max_prefix_len + W
 * masks      uint64 [B][R] (bits >= W are ignored)
 * B >= 0; 1 <= R <= 64; 0 <= W <= 64; Hq % Hkv == 0; D in {64, 128}
 * dtype      TAV_BF16 (bf16 MFMA prefix, fp32 accumulation), TAV_F32
 *            (fp32 vector-ALU path) or TAV_FP8_E4M3: an unscaled FP8 E4M3
 *            K/V cache with a bf16 query ([DTS] "One tree attention ...": FP8
 *            leaves the cascade's structure as it is; the prefix decode
 *            rounds the query to FP8, the window part keeps it unrounded and
 *            widens the window's keys and values).  Prefix keys are scored with the
 *            query rounded to the nearest E4M3 value (ties to even,
 *            saturating at +-448), window keys with the bf16 query; keys
 *            and values are widened exactly to bf16, so every product is
 *            exact and sums in fp32.  Strides count elements (bytes for
 *            FP8).
 * out        [B][R][Hq][D] in q's dtype (bf16 rounded to nearest even)
 * lse2       float [B][R][Hq] or NULL: log2 of the sum over visible keys of
 *            exp(score) (so 2^lse2 is the softmax denominator)
 * workspace  device memory of >= tree_attention_workspace_size(...) bytes,
 *            256-byte aligned; contents are scratch between calls
 */
tav_status tree_attention(const void *q, const void *k_cache, const void *v_cache,
                          tav_dtype dtype, int64_t stride_page, int64_t stride_head,
                          int64_t stride_token, int64_t num_pages,
                          const int32_t *page_table, int32_t max_pages, int32_t page_size,
                          const int32_t *prefix_len, int32_t max_prefix_len,
                          int32_t prefix_window, const uint64_t *masks, int32_t W,
                          int32_t B, int32_t R, int32_t Hq, int32_t Hkv, int32_t D,
                          float sm_scale, void *out, float *lse2, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * The two phases of tree_attention as separate calls, with tree_attention's
 * arguments and contract; tree_attention is exactly tree_attention_prefix
 * followed by tree_attention_window_merge on the same stream and workspace,
 * and the two calls must get the same arguments.  They mirror the cascade's
 * split ([DTS] "One tree attention ...": the prefix decode, then the window
 * part and the merge), so a caller can place other work between them or
 * time them apart.
 *   tree_attention_prefix        reads q, the K/V prefix pages, page_table and
 *                                prefix_len; writes the split-K prefix partials
 *                                into the workspace
 *   tree_attention_window_merge  reads the workspace partials of a preceding
 *                                tree_attention_prefix with the same arguments,
 *                                the window keys and masks; writes out and lse2
 * Except: when the prefix runs as a single split over bf16 K/V with at most
 * 32 or more than 128 folded rows per kv head (R x Hq / Hkv; the library
 * picks the split count from B, Hkv and the prefix length), and out and,
 * for W > 0, masks are given, tree_attention_prefix also attends the window
 * keys and writes out and lse2 itself, and tree_attention_window_merge then
 * launches nothing.
 * The window keys are then one more stage of the prefix launch, with the
 * same semantics (a non-finite V value reaches exactly the rows that see
 * its key).
 */
tav_status tree_attention_prefix(const void *q, const void *k_cache, const void *v_cache,
                                 tav_dtype dtype, int64_t stride_page, int64_t stride_head,
                                 int64_t stride_token, int64_t num_pages,
                                 const int32_t *page_table, int32_t max_pages, int32_t page_size,
                                 const int32_t *prefix_len, int32_t max_prefix_len,
                                 int32_t prefix_window, const uint64_t *masks, int32_t W,
                                 int32_t B, int32_t R, int32_t Hq, int32_t Hkv, int32_t D,
                                 float sm_scale, void *out, float *lse2, void *workspace,
                                 size_t workspace_bytes, void *stream);
tav_status tree_attention_window_merge(const void *q, const void *k_cache, const void *v_cache,
                                       tav_dtype dtype, int64_t stride_page, int64_t stride_head,
                                       int64_t stride_token, int64_t num_pages,
                                       const int32_t *page_table, int32_t max_pages,
                                       int32_t page_size, const int32_t *prefix_len,
                                       int32_t max_prefix_len, int32_t prefix_window,
                                       const uint64_t *masks, int32_t W, int32_t B, int32_t R,
                                       int32_t Hq, int32_t Hkv, int32_t D, float sm_scale,
                                       void *out, float *lse2, void *workspace,
                                       size_t workspace_bytes, void *stream);

/*
 * tree_attention without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): the split-K partials live in a fixed device
 * array of TAV_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends.  Arguments, outputs and errors are
 * tree_attention's, minus workspace and workspace_bytes; the call allocates
 * nothing and launches the same kernels.
 *   Limit: shapes whose partials (tree_attention_workspace_size) exceed
 *   TAV_NOALLOC_SCRATCH_BYTES are refused with TAV_ERR_WORKSPACE before
 *   anything is launched (long-context B 4, R 64, Hq 32, D 128 needs about
 *   38 MB; B 32, R 64, Hq 64 about 135 MB and is refused).
 *   Sharing: every call on one GPU uses that GPU's one array, which keeps
 *   the last call's partials; calls that overlap on one GPU (other streams,
 *   other threads) race and must be serialised by the caller.  No part of
 *   the array needs to start at zero: each call writes every partial it
 *   reads before reading it.
 *   The first call on a GPU resolves the array's address there (with that
 *   GPU made current for the lookup) and may return TAV_ERR_HIP if that
 *   fails.
 */
#define TAV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
tav_status tree_attention_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                  tav_dtype dtype, int64_t stride_page, int64_t stride_head,
                                  int64_t stride_token, int64_t num_pages,
                                  const int32_t *page_table, int32_t max_pages,
                                  int32_t page_size, const int32_t *prefix_len,
                                  int32_t max_prefix_len, int32_t prefix_window,
                                  const uint64_t *masks, int32_t W, int32_t B, int32_t R,
                                  int32_t Hq, int32_t Hkv, int32_t D, float sm_scale,
                                  void *out, float *lse2, void *stream);

/*
 * Greedy tree verify ([MEM] "Walking the accepted path"): from the root, move
 * to the child whose draft token matches the target's argmax at the current
 * node; stop when no child matches.  Ties between children carrying the same
 * token go to the lowest node index.  The walk takes at most N nodes.
 *
 * draft_tokens, target_argmax, parents  int32 [B][N]; B >= 0; 1 <= N <= 64
 * accepted_path   int32 [B][N] out: node indices, -1 padded
 *                 (the single owner of the path, [DTS] "The tree is a
 *                 parameter of the chain path")
 * accept_len      int32 [B] out: nodes on the path, counting the root
 *                 ([ETA] section 2: accept_lens = correct drafts + 1)
 * accepted_tokens int32 [B][N] or NULL: out target_argmax[path[k]] for
 *                 k < accept_len (the last is the bonus token), -1 after
 */
tav_status verify_tree_greedy(const int32_t *draft_tokens, const int32_t *target_argmax,
                              const int32_t *parents, int32_t B, int32_t N,
                              int32_t *accepted_path, int32_t *accept_len,
                              int32_t *accepted_tokens, void *stream);

/*
 * One row table for compact_window_rows: a buffer holding, per (request,
 * window slot), n_heads segments of row_bytes bytes (e.g. one layer's K cache
 * with n_heads = Hkv and row_bytes = D * element size, or a hidden-state
 * buffer with n_heads = 1).  All strides are in BYTES.
 *   paged (page_table != NULL): window slot i of request b is logical
 *     position prefix_len[b] + i; segment h of it is at
 *     base + page*stride_page + h*stride_head + (pos % page_size)*stride_token
 *     with page = page_table[b*max_pages + pos / page_size]
 *   dense (page_table == NULL): at base + b*stride_batch + i*stride_token
 *     + h*stride_head
 * row_bytes, the strides and base must be multiples of 4.  Each physical
 * region must appear in at most one table of a call ([DTS] "Recurrent state
 * follows the parent": each region moves once per cache group).
 */
typedef struct {
    void *base;
    const int32_t *page_table; /* device int32 [B][max_pages], or NULL */
    const int32_t *prefix_len; /* device int32 [B] (paged tables)       */
    int32_t max_pages;
    int32_t page_size;         /* power of two in [1, 1024] (paged)     */
    int64_t num_pages;         /* pages in the pool (paged), for bounds */
    int64_t stride_page;
    int64_t stride_token;
    int64_t stride_head;
    int64_t stride_batch;      /* dense tables */
    int32_t n_heads;
    int32_t row_bytes;
} tav_rows;

/*
 * Moves the accepted path's rows to the window's leading slots in every
 * table: for i < accept_len[b], row i <- row accepted_path[b][i], copied as
 * 32-bit words so any element type works ([DTS] "The tree is a parameter of
 * the chain path": compact_window_rows copies words; [MEM] "Discarding the
 * rejected branches' KV").  Every source row of a request is read before any
 * row is written, so overlapping paths such as [0, 2, 5] are safe.  Rows at
 * or past accept_len, other requests and other bytes are not touched.
 *
 * tables   HOST array of n_tables descriptors (copied at call time)
 * accepted_path int32 [B][N], accept_len int32 [B] (device, e.g. from
 *          verify_tree_greedy).  accept_len is clamped to [0, N]; a path
 *          entry outside [0, N), or a row whose page falls outside the table,
 *          is skipped.
 * B >= 0; 1 <= N <= 64; 0 <= n_tables
 */
tav_status compact_window_rows(const tav_rows *tables, int32_t n_tables,
                               const int32_t *accepted_path, const int32_t *accept_len,
                               int32_t B, int32_t N, void *stream);

/*
 * Sampled verify ([DTS] "Sampled verify keys noise by position"): the target
 * token of every verify row drawn by Gumbel-max, keyed by (seed of the
 * request, the position the node predicts) -- positions[b][i] + 1, where
 * positions is vc + depth as tree_build_masks writes it -- never by the row,
 * so siblings share their noise and a chain row draws what plain decoding
 * draws at that position.  Acceptance is then verify_tree_greedy with these
 * tokens as target_argmax (a child is accepted when it equals its parent's
 * draw).
 *
 * Noise: Philox4x32-10 (Salmon et al., "Parallel Random Numbers: As Easy as
 * 1, 2, 3", SC 2011; the pages name no generator) at counter {v / 4, key
 * position, 0, 0} under key {seed & 0xffffffff, seed >> 32}; word v % 4 of
 * token v, top 24 bits b: u = (b + 1/2) / 2^24, g = -ln(-ln u).
 * z_v = logits[v] / T + g_v in fp32; token = argmax_v z_v, the lowest v on
 * ties, NaN ranking last (a row of -inf / NaN only gives token 0).
 * T = temperature[b]; T <= 0 (or NaN) takes the argmax of the logits.
 *
 * logits      device [B][N][row_stride] elements of dtype (TAV_BF16 or
 *             TAV_F32), V used per row; 16-byte aligned, row_stride >= V and
 *             row_stride * element size a multiple of 16 bytes
 * temperature device float [B]; seed device uint64 [B]
 * positions   device int32 [B][N]
 * tokens      device int32 [B][N] out
 * workspace   device memory of >= tree_sample_workspace_size(B, N, V)
 *             bytes, 256-byte aligned; scratch between calls
 * B >= 0; 1 <= N <= 64; V >= 1
 */
size_t tree_sample_workspace_size(int32_t B, int32_t N, int32_t V);
tav_status tree_sample_gumbel(const void *logits, tav_dtype dtype, int64_t row_stride, int32_t V,
                              int32_t B, int32_t N, const float *temperature,
                              const uint64_t *seed, const int32_t *positions, int32_t *tokens,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * Sampled verify by tree rejection sampling ([DDT] "The Implementation": a
 * node's children are tried in descending draft probability and the first
 * one passing the rejection test is accepted; [DTS] "Sampled verify keys
 * noise by position": recursive rejection sampling is exact in
 * distribution).  The draft tokens are fixed candidates.  At node cur,
 * w(v) = probs[cur][v] where positive and finite (else 0), S = sum_v w(v),
 * and R holds the tokens rejected so far at cur, of total weight E.  Child c
 * (token x) is accepted when
 *     coins[c] * (S - E) < w(x)      (0 when x is outside [0, V) or in R),
 * i.e. with the residual's probability of x; otherwise x joins R.  Children
 * are the nodes with parents[c] == cur, in descending draft_score, the lower
 * index on ties (index order when draft_score is NULL).  An accepted child
 * continues the walk.  When none is (or the path holds N nodes) the walk
 * stops and the bonus token is drawn from the residual r = w without R: the
 * lowest v whose running sum of r exceeds bonus_u[cur] * sum_v r(v) (the
 * last v of positive residual if rounding leaves none; token 0 if r is all
 * zero).  The token emitted at every depth is then distributed as the
 * target row there.
 *
 * With draft_q given, the children are tested against the draft
 * distribution that drew them ([DTS] "Sampled verify keys noise by
 * position": recursive rejection sampling against the draft q of a node's
 * children).  At node cur the residual starts as r = w / S, q^ = q / Q with
 * q = draft_q[cur] (positive finite entries) and Q its total; child c (token
 * x) is accepted when coins[c] * q^(x) < r(x), probability min(1, r(x) /
 * q^(x)); otherwise r becomes max(0, r - q^) renormalised (all zero when
 * nothing is left).  The bonus is drawn from the final r as above.  This is
 * exact when the children are independent draws from q tested in an order
 * that does not depend on the drawn tokens.
 *
 * Sums are fp32 in a fixed order (tiles of 256 tokens, slices of 64 tiles,
 * the slices in order), so a decision within rounding of a tie may differ
 * from an exact evaluation; the outcome is the same on every run.  Where
 * fp32 rounding leaves the bonus draw's running sum short of the target at
 * a level of its search (slice, tile, token), the last positive entry of
 * that level is taken.
 *
 * probs        device fp32 [B][N][row_stride], V used per row: the target
 *              distribution after the node (softmax at the sampling
 *              temperature; rows need not sum to 1); 16-byte aligned,
 *              row_stride >= V and a multiple of 4
 * draft_q      device fp32 [B][N][q_row_stride] or NULL: row n is the draft
 *              distribution that drew node n's children; 16-byte aligned,
 *              q_row_stride >= V and a multiple of 4
 * draft_tokens, parents  int32 [B][N] (parents[0] = -1 is the root)
 * draft_score  fp32 [B][N] or NULL: the sibling order (e.g. the draft
 *              probability of each node's token)
 * coins, bonus_u  fp32 [B][N], uniform in [0, 1): the coin of each node's
 *              test and the bonus draw at the node where the walk stops
 * accepted_path, accept_len, accepted_tokens as verify_tree_greedy; the
 *              tokens are draft[path[k + 1]] for k + 1 < accept_len and the
 *              bonus at k = accept_len - 1 (NULL to skip)
 * workspace    device, >= verify_tree_rejection_workspace_size(B, N, V)
 *              bytes, 256-byte aligned; owned by the caller, cleared and
 *              used by the call (the slice totals and tile sums of the
 *              workgroups that share a request's row passes), so calls that
 *              may overlap need workspaces of their own
 * B >= 0; 1 <= N <= 64; 1 <= V <= 2^20
 * The workgroups of a request wait for one another's slice totals in the
 * workspace, each wait bounded; should one give up, the request reports
 * accept_len -1 and a path of -1.
 */
size_t verify_tree_rejection_workspace_size(int32_t B, int32_t N, int32_t V);
tav_status verify_tree_rejection(const float *probs, int64_t row_stride, int32_t V,
                                 const float *draft_q, int64_t q_row_stride,
                                 const int32_t *draft_tokens, const int32_t *parents,
                                 const float *draft_score, const float *coins,
                                 const float *bonus_u, int32_t B, int32_t N,
                                 int32_t *accepted_path, int32_t *accept_len,
                                 int32_t *accepted_tokens, void *workspace,
                                 size_t workspace_bytes, void *stream);

/*
 * Prefix, window and merge as in tree_attention, over an MLA latent cache ([DTS] "One tree attention ...",
 * the MLA paragraph).  Each token stores one latent row, shared by every
 * query head: its first Dc channels (kv_lora_rank) meet the query's first Dc
 * channels in the score and are also the value; its Dr rotary channels
 * after them meet the query's last Dr channels (Dr = 0: no rotary part).
 * Visibility as tree_attention (the whole prefix, plus window node j at
 * logical position P + j for the set bits j < W of the row's mask).
 *   s_t = sm_scale * (q[:Dc] . c_t + q[Dc:] . r_t),  out = softmax(s) . c,
 *   lse2 = log2 sum_t exp(s_t)
 * q          [B][R][Hq][Dc + Dr] bf16 (the absorbed query)
 * latent     paged pool: the row of logical position t is at element
 *            page_table[b][t / page_size] * stride_page + (t % page_size) *
 *            stride_token, Dc + Dr contiguous elements of type dtype
 *            (latent part, then the rotary part); strides in elements,
 *            rows 16-byte aligned
 * dtype      TAV_BF16, or TAV_FP8_E4M3 for a cache of unscaled OCP E4M3
 *            codes: the page hands the absorbed query over in FP8 under an
 *            FP8 cache and the window kernel widens it back exactly, so
 *            every key, prefix and window, is scored with q rounded to the
 *            nearest E4M3 value (ties to even, +-448 saturation); products
 *            are then exact, sums fp32, and the value is the widened latent
 * page_table, prefix_len, max_prefix_len, masks, W, B, R as tree_attention
 * Dc == 512; Dr in {0, 64}; page_size a power of two <= 1024
 * sm_scale   <= 0 selects 1/sqrt(Dc + Dr)
 * out        [B][R][Hq][Dc] bf16 (round to nearest even); lse2 float
 *            [B][R][Hq] or NULL
 * workspace  >= tree_attention_mla_workspace_size(...) bytes, 256-byte
 *            aligned; scratch between calls
 */
size_t tree_attention_mla_workspace_size(int32_t B, int32_t R, int32_t Hq, int32_t Dc,
                                         int32_t Dr, int32_t max_prefix_len, int32_t page_size);
tav_status tree_attention_mla(const void *q, const void *latent, tav_dtype dtype,
                              int64_t stride_page, int64_t stride_token, int64_t num_pages,
                              const int32_t *page_table, int32_t max_pages, int32_t page_size,
                              const int32_t *prefix_len, int32_t max_prefix_len,
                              const uint64_t *masks, int32_t W, int32_t B, int32_t R, int32_t Hq,
                              int32_t Dc, int32_t Dr, float sm_scale, void *out, float *lse2,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * Tree construction, the step before the verify path.  Candidate order: the
 * higher score first, the lower candidate id on equal scores, NaN after
 * every number ([DTS] "Tree construction is deterministic").
 *
 * tree_beam_step: one EAGLE-2 expansion ([MEM] "EAGLE-2: the tree stops
 * being a constant": the surviving paths' cumulative scores times the new
 * conditional probabilities, the topk best paths kept; [ETA] "candidate pool
 * to verify rows": cumulative path scores, e.g. 0.60 x 0.70 = 0.42).
 *   scores     float [B][n_surv]: the survivors' cumulative scores (1 for
 *              the root at the first step)
 *   surv_idx   int32 [B][n_surv]: their pool indices (-1 for the root)
 *   child_p    float [B][n_surv][K]: each survivor's children's conditional
 *              probabilities; child_tok int32 [B][n_surv][K] their tokens
 *   pool_*     [B][C] candidate pool; entries pool_base + s*K + j are written:
 *              score scores[s] * child_p[s][j] (fp32 product), parent
 *              surv_idx[s], token child_tok[s][j]
 *   next_scores float [B][K], next_idx int32 [B][K] out: the K best children
 *              (flat index s*K + j as the id), best first, as pool indices.
 *              They may be the scores / surv_idx buffers (every input is read
 *              before any output is written).
 *   1 <= n_surv, K; n_surv * K <= 1024; pool_base + n_surv * K <= C
 *
 * tree_select_candidates: the verify tree from a request's pool ([MEM]
 * organize_draft_results: the num_draft_token - 1 best of the flattened
 * pool, sorted, tokens gathered, parent topology kept; [ETA] "the verify root
 * is not an ordinary draft candidate": the previous bonus token is node 0).
 *   pool_scores float [B][C], pool_parents int32 [B][C] (-1 = root; a parent
 *              must precede its child), pool_tokens int32 [B][C]
 *   root_tokens int32 [B]
 *   order      0: nodes in pool order; 1: depth-first order visiting a
 *              node's higher-scoring child first ([DTS]: the top path is
 *              then numbered 0, 1, 2, ...)
 *   parents, tokens int32 [B][N] out: the tree (parents[i] < i) and its
 *              tokens; selected int32 [B][N] out: each node's pool index (-1
 *              for the root)
 *   tree_error int32 [B] or NULL out: 0, or 1 + the first node (pool order)
 *              whose parent is not kept or does not precede it ([MEM]: a
 *              missing parent is rejected, never treated as a root); that
 *              request's outputs are then -1
 *   1 <= N <= 64; max(1, N - 1) <= C <= 8192
 *
 * tree_retrieve_links: first-child / next-sibling arrays in node order
 * ([MEM] "Flattening, and the two link arrays"; [DDT] compile_ddtree_retrieve)
 *   parents int32 [B][N]; next_token, next_sibling int32 [B][N] out (-1 =
 *   none).  1 <= N <= 64
 */
tav_status tree_beam_step(const float *scores, const int32_t *surv_idx, const float *child_p,
                          const int32_t *child_tok, int32_t B, int32_t n_surv, int32_t K,
                          int32_t C, int32_t pool_base, float *pool_scores,
                          int32_t *pool_parents, int32_t *pool_tokens, float *next_scores,
                          int32_t *next_idx, void *stream);
tav_status tree_select_candidates(const float *pool_scores, const int32_t *pool_parents,
                                  const int32_t *pool_tokens, const int32_t *root_tokens,
                                  int32_t B, int32_t C, int32_t N, int32_t order,
                                  int32_t *parents, int32_t *tokens, int32_t *selected,
                                  int32_t *tree_error, void *stream);
tav_status tree_retrieve_links(const int32_t *parents, int32_t B, int32_t N,
                               int32_t *next_token, int32_t *next_sibling, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TREEVERIFY_H */
