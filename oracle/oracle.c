/*
 * Plain CPU fp64 oracle for the draft-tree verify path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP library; every routine below is the plain definition
 * of what the method computes, written out slowly and in the order the pages
 * state it, with no blocking, fusion or reordering beyond that.
 *
 * Sources (page title, section):
 *  [DTS]  "Draft-tree speculation" (tokenspeed design notes)
 *  [ETA]  "EAGLE Tree Attention candidate layout, positions and visibility"
 *         (SGLang EAGLE tree-verify analysis, Chinese)
 *  [MEM]  "Medusa, EAGLE-1/2/3, MTP, and tree attention" (course chapter)
 *  [DDT]  "From Greedy to Sampling: The Architecture of Choice in DDTree
 *         Speculative Decoding"
 *
 * Floating point: every score, exponential, sum and output is fp64, on the
 * exact input values (bf16 inputs are widened bit-exactly).  Parity of every
 * routine here is pinned by tests against worked values printed on the
 * pages, closed forms, brute force and a library attention routine; see the
 * test module for the list.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD 1

/* ------------------------------------------------------------------ */
/* element access                                                      */
/* ------------------------------------------------------------------ */

/*
 * dtype codes of this file: 0 = fp32, 1 = bf16 (raw 16-bit patterns),
 * 2 = FP8 E4M3 (raw bytes).  E4M3 here is the OCP 8-bit format with 1 sign,
 * 4 exponent (bias 7) and 3 mantissa bits, no infinities, and NaN for
 * exponent and mantissa all ones; it is the unscaled FP8 KV cache format of
 * [DTS] "One tree attention ..." (an FP8 E4M3 cache changes no structure).
 */
static double orc_e4m3(uint8_t b)
{
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);            /* subnormal: m/8 * 2^(1-7) */
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

static double orc_load(const void *base, int dtype, int64_t idx)
{
    if (dtype == 0)
        return (double)((const float *)base)[idx];
    if (dtype == 2)
        return orc_e4m3(((const uint8_t *)base)[idx]);
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Exposed for the pins: the decoded value of one E4M3 code. */
double orc_e4m3_decode(int code)
{
    return orc_e4m3((uint8_t)code);
}

/*
 * x rounded to the nearest E4M3 value, ties to the even code (mantissa LSB
 * 0); magnitudes past the largest finite value (448) give +-448, NaN stays
 * NaN.  Written as a search over the 127 non-negative finite codes, whose
 * values increase with the code.  This is the cast of the query that the
 * prefix half of the cascade takes under an FP8 cache ([DTS] "One tree
 * attention ...": the leaf's decode rounds the query to FP8, the window
 * part keeps it unrounded).
 */
double orc_e4m3_round(double x)
{
    if (isnan(x))
        return NAN;
    double a = fabs(x) > 448.0 ? 448.0 : fabs(x), best = 0.0, err = INFINITY;
    int best_code = 0;
    for (int c = 0; c < 127; ++c) {
        double v = orc_e4m3((uint8_t)c), e = fabs(v - a);
        if (e < err || (e == err && (c & 1) == 0 && (best_code & 1) == 1)) {
            err = e;
            best = v;
            best_code = c;
        }
    }
    return x < 0 || (x == 0 && signbit(x)) ? -best : best;
}

/* ------------------------------------------------------------------ */
/* tree metadata                                                       */
/* ------------------------------------------------------------------ */

/*
 * Ancestor masks, depth and RoPE positions of every node.
 *
 * [ETA] section 1 (the visibility rule M(i,j)): row i sees key j of the
 * window iff j == i or j is an ancestor of i.  The bit form follows
 * [DTS] "One tree attention ...": one 64-bit ancestor mask per row, bit j
 * standing for window node j.  The walk up the parent links is the one of
 * [MEM]'s tiny numpy reference (climb while the ancestor is not -1).
 * Depth counts the climbs; the position is the prefix length plus depth
 * ([ETA] section 2, positions = seq_len + depth; [DTS] "Position follows
 * depth, slot follows node index": node i sits at vc + depth[i]).
 *
 * A tree is valid when node 0 is the only root (parent -1) and every other
 * node's parent is an earlier node ([ETA] section 1 puts the root first;
 * [MEM] "Building the mask, for real": a missing parent is rejected, never
 * treated as a root).  For an invalid request tree_error[b] = 1 + the first
 * offending node, and its masks are 0, depth and positions -1.
 */
int orc_build_masks(const int32_t *parents, int B, int N, const int32_t *vc,
                    int32_t *depth, uint64_t *masks, int32_t *positions,
                    int32_t *tree_error)
{
    if (B < 0 || N < 1 || N > 64)
        return ORC_BAD;
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parents + (int64_t)b * N;
        int bad = -1;
        for (int i = 0; i < N && bad < 0; ++i) {
            if (i == 0 && par[0] != -1)
                bad = 0;
            if (i > 0 && (par[i] < 0 || par[i] >= i))
                bad = i;
        }
        if (tree_error)
            tree_error[b] = bad < 0 ? 0 : 1 + bad;
        for (int i = 0; i < N; ++i) {
            int64_t o = (int64_t)b * N + i;
            if (bad >= 0) {
                masks[o] = 0;
                depth[o] = -1;
                if (positions)
                    positions[o] = -1;
                continue;
            }
            uint64_t m = 0;
            int climbs = 0;
            int a = i;
            while (a != -1) {
                m |= (uint64_t)1 << a;
                a = par[a];
                if (a != -1)
                    ++climbs;
            }
            masks[o] = m;
            depth[o] = climbs;
            if (positions)
                positions[o] = (vc ? vc[b] : 0) + climbs;
        }
    }
    return ORC_OK;
}

/*
 * Position shifts of [DTS] "Position follows depth, slot follows node
 * index": load_step moves window row i from vc + i to vc + depth[i]
 * (direction +1); compact_rows moves it back (direction -1).
 */
int orc_shift_positions(int32_t *pos, const int32_t *depth, int B, int N,
                        int direction)
{
    if (direction != 1 && direction != -1)
        return ORC_BAD;
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < N; ++i) {
            int64_t o = (int64_t)b * N + i;
            pos[o] += direction * (depth[o] - i);
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* attention                                                           */
/* ------------------------------------------------------------------ */

/*
 * Softmax attention of one query row over an ordered list of keys, in fp64.
 * s_t = scale * sum_d q[d] k_t[d], where the first nq8 keys take q rounded
 * to E4M3 (orc_e4m3_round) instead of q;  m = max s;  Z = sum exp(s_t - m);
 * o = sum exp(s_t - m) v_t / Z;  lse2 = (m + ln Z) / ln 2, the base-2
 * log-sum-exp of the scores ([DTS] "One tree attention ...": both halves of
 * the cascade carry a base-2 log-sum-exp).  No key: o = 0, lse2 = -inf.
 * kofs/vofs hold the element offset of each key's row.
 */
static void orc_softmax_row(const void *qb, int64_t qofs, const void *kb,
                            const void *vb, int qdt, int kvdt, const int64_t *kofs,
                            int nk, int nq8, int D, double scale, double *s,
                            double *out, double *lse2)
{
    for (int d = 0; d < D; ++d)
        out[d] = 0.0;
    if (nk == 0) {
        *lse2 = -INFINITY;
        return;
    }
    double *qv = (double *)malloc(sizeof(double) * 2 * D), *q8 = qv + D;
    for (int d = 0; d < D; ++d) {
        qv[d] = orc_load(qb, qdt, qofs + d);
        q8[d] = orc_e4m3_round(qv[d]);
    }
    double m = -INFINITY;
    for (int t = 0; t < nk; ++t) {
        const double *qq = t < nq8 ? q8 : qv;
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
            acc += qq[d] * orc_load(kb, kvdt, kofs[t] + d);
        s[t] = scale * acc;
        if (s[t] > m)
            m = s[t];
    }
    double Z = 0.0;
    for (int t = 0; t < nk; ++t) {
        double w = exp(s[t] - m);
        Z += w;
        for (int d = 0; d < D; ++d)
            out[d] += w * orc_load(vb, kvdt, kofs[t] + d);
    }
    for (int d = 0; d < D; ++d)
        out[d] /= Z;
    *lse2 = (m + log(Z)) / log(2.0);
    free(qv);
}

/*
 * Tree attention over a paged KV cache.
 *
 * Row r of request b, query head h, reads kv head h / (Hq / Hkv).  Its
 * visible keys, in this order, are
 *   - the committed prefix: logical positions t in [p_lo, P), where P =
 *     prefix_len[b] and p_lo = max(0, P - prefix_window) when
 *     prefix_window > 0, else 0 ([ETA] section 1: every row sees the
 *     committed prefix; [DTS] "One tree attention ...": a draft layer with
 *     a sliding window sees it as it stood at the end of the round's prefix);
 *   - then window node j, stored at logical position P + j, for j < W in
 *     ascending order with bit j of masks[b*R + r] set ([DTS] "One tree
 *     attention ...": the 64-bit ancestor mask covers the last W keys;
 *     "Position follows depth, slot follows node index": the slot follows
 *     the node index).
 * Logical position t lives in physical page page_table[b*max_pages + t/ps]
 * at slot t % ps; the element offset of (page, kv head g, slot) is
 * page*stride_page + g*stride_head + slot*stride_token, channels contiguous.
 * Keys that are not visible are never read.
 *
 * q holds dtype elements, k_cache and v_cache kv_dtype elements.  An FP8
 * cache takes a bf16 query: prefix keys are scored with the query rounded
 * to E4M3, window keys with the bf16 query itself ([DTS] "One tree
 * attention ...": the leaf's decode rounds the query to FP8, while the
 * window part keeps the query unrounded and converts the window's FP8 keys
 * and values once loaded).
 * rows: optional list of flat row ids ((b*R + r)*Hq + h); out/lse2 then hold
 * n_rows entries in list order.  With rows == NULL every row is computed and
 * out is [B][R][Hq][D], lse2 [B][R][Hq].
 * q is [B][R][Hq][D] contiguous.  sm_scale <= 0 means 1/sqrt(D).
 */
int orc_tree_attention(const void *q, const void *k_cache, const void *v_cache,
                       int dtype, int kv_dtype, int64_t stride_page, int64_t stride_head,
                       int64_t stride_token, const int32_t *page_table,
                       int max_pages, int page_size, const int32_t *prefix_len,
                       int prefix_window, const uint64_t *masks, int W, int B,
                       int R, int Hq, int Hkv, int D, double sm_scale,
                       const int64_t *rows, int64_t n_rows, double *out,
                       double *lse2)
{
    if (Hkv <= 0 || Hq % Hkv != 0 || W < 0 || W > 64 || page_size <= 0)
        return ORC_BAD;
    if (sm_scale <= 0.0)
        sm_scale = 1.0 / sqrt((double)D);
    int64_t total = rows ? n_rows : (int64_t)B * R * Hq;
    int group = Hq / Hkv;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t n = 0; n < total; ++n) {
        int64_t id = rows ? rows[n] : n;
        int h = (int)(id % Hq);
        int r = (int)((id / Hq) % R);
        int b = (int)(id / ((int64_t)Hq * R));
        int g = h / group;
        int P = prefix_len[b];
        int p_lo = prefix_window > 0 && P > prefix_window ? P - prefix_window : 0;
        int nk_max = P - p_lo + W;
        int64_t *kofs = (int64_t *)malloc(sizeof(int64_t) * (nk_max > 0 ? nk_max : 1));
        double *s = (double *)malloc(sizeof(double) * (nk_max > 0 ? nk_max : 1));
        int nk = 0, nq8 = 0;
        uint64_t m = masks[(int64_t)b * R + r];
        for (int t = p_lo; t < P + W; ++t) {
            if (t >= P) {
                int j = t - P;
                if (!((m >> j) & 1))
                    continue;
            }
            int lp = t / page_size;
            if (lp >= max_pages) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            int64_t page = page_table[(int64_t)b * max_pages + lp];
            kofs[nk++] = page * stride_page + (int64_t)g * stride_head +
                         (int64_t)(t % page_size) * stride_token;
            if (t < P && kv_dtype == 2)
                nq8 = nk;
        }
        int64_t qofs = (((int64_t)b * R + r) * Hq + h) * D;
        orc_softmax_row(q, qofs, k_cache, v_cache, dtype, kv_dtype, kofs, nk, nq8, D,
                        sm_scale, s, out + n * D, lse2 + n);
        free(kofs);
        free(s);
    }
    return bad ? ORC_BAD : ORC_OK;
}

/*
 * Plain causal attention on contiguous keys: q is [n][Hq][D], k and v are
 * [L][Hkv][D].  Query row i sits at position L - n + i and sees keys
 * t <= L - n + i, in ascending order.  Used by the pins: a chain tree must
 * equal this ([DTS] "The tree is a parameter of the chain path": the chain
 * is the special tree with parent[i] = i - 1), and each tree row must equal the last row of
 * this run on prefix + its own root-to-node path ([ETA] section 1,
 * L(v) = Target(prefix + path(root -> v))).
 */
int orc_causal_attention(const void *q, const void *k, const void *v,
                         int dtype, int n, int L, int Hq, int Hkv, int D,
                         double sm_scale, double *out, double *lse2)
{
    if (Hkv <= 0 || Hq % Hkv != 0 || n > L)
        return ORC_BAD;
    if (sm_scale <= 0.0)
        sm_scale = 1.0 / sqrt((double)D);
    int group = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t id = 0; id < (int64_t)n * Hq; ++id) {
        int i = (int)(id / Hq), h = (int)(id % Hq), g = h / group;
        int nk = L - n + i + 1;
        int64_t *kofs = (int64_t *)malloc(sizeof(int64_t) * nk);
        double *s = (double *)malloc(sizeof(double) * nk);
        for (int t = 0; t < nk; ++t)
            kofs[t] = ((int64_t)t * Hkv + g) * D;
        orc_softmax_row(q, id * D, k, v, dtype, dtype, kofs, nk, 0, D, sm_scale, s,
                        out + id * D, lse2 + id);
        free(kofs);
        free(s);
    }
    return ORC_OK;
}

/*
 * Merge of softmax states over disjoint key sets ([ETA] section 4, the
 * cascade merge): with Z_k the unnormalised weight sum of part k (here
 * Z_k = 2^lse2_k), O = sum_k Z_k O_k / sum_k Z_k and lse2 = log2 sum_k Z_k.
 * Parts with lse2 = -inf (no key) carry no weight; if every part is empty the
 * result is O = 0, lse2 = -inf.  o_parts is [S][n][D], lse2_parts [S][n].
 */
int orc_merge(const double *o_parts, const double *lse2_parts, int S, int n,
              int D, double *out, double *lse2)
{
    for (int i = 0; i < n; ++i) {
        double mx = -INFINITY;
        for (int k = 0; k < S; ++k)
            if (lse2_parts[(int64_t)k * n + i] > mx)
                mx = lse2_parts[(int64_t)k * n + i];
        for (int d = 0; d < D; ++d)
            out[(int64_t)i * D + d] = 0.0;
        if (mx == -INFINITY) {
            lse2[i] = -INFINITY;
            continue;
        }
        double Zsum = 0.0;
        for (int k = 0; k < S; ++k) {
            double l = lse2_parts[(int64_t)k * n + i];
            if (l == -INFINITY)
                continue;
            double Z = exp2(l - mx); /* Z_k scaled by 2^-mx */
            Zsum += Z;
            for (int d = 0; d < D; ++d)
                out[(int64_t)i * D + d] += Z * o_parts[((int64_t)k * n + i) * D + d];
        }
        for (int d = 0; d < D; ++d)
            out[(int64_t)i * D + d] /= Zsum;
        lse2[i] = mx + log2(Zsum);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* greedy verify                                                       */
/* ------------------------------------------------------------------ */

/*
 * Greedy tree walk ([MEM] "Walking the accepted path"): start at the root;
 * t = target_argmax[cur], the target's token at the current node; move to a
 * child of cur whose draft token equals t; stop when none does.  When
 * several children carry t, the lowest node index wins (the pages' walk
 * scans children in order; [DTS] "Tree construction is deterministic"
 * numbers the best child first).  accept_len counts the root ([ETA]
 * section 2, accept_lens = num_correct_drafts + 1; [DDT]: the accepted
 * count includes the root).  path is N wide and -1 padded; tokens[k] =
 * target_argmax[path[k]] for k < accept_len (the last one is the bonus),
 * -1 after.  The walk takes at most N nodes whatever the parent array holds.
 */
int orc_verify_greedy(const int32_t *draft, const int32_t *target,
                      const int32_t *parents, int B, int N, int32_t *path,
                      int32_t *accept_len, int32_t *tokens)
{
    if (N < 1 || N > 64)
        return ORC_BAD;
    for (int b = 0; b < B; ++b) {
        const int32_t *dr = draft + (int64_t)b * N;
        const int32_t *tg = target + (int64_t)b * N;
        const int32_t *par = parents + (int64_t)b * N;
        int32_t *pb = path + (int64_t)b * N;
        for (int k = 0; k < N; ++k)
            pb[k] = -1;
        int len = 0;
        int cur = 0;
        pb[len++] = cur;
        while (len < N) {
            int t = tg[cur];
            int next = -1;
            for (int c = 0; c < N; ++c)
                if (par[c] == cur && dr[c] == t) {
                    next = c;
                    break;
                }
            if (next < 0)
                break;
            cur = next;
            pb[len++] = cur;
        }
        accept_len[b] = len;
        if (tokens)
            for (int k = 0; k < N; ++k)
                tokens[(int64_t)b * N + k] = k < len ? tg[pb[k]] : -1;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* compaction                                                          */
/* ------------------------------------------------------------------ */

/*
 * One row table of the compaction: a buffer with one row of n_heads
 * segments of row_bytes bytes per (request, window slot).  Paged tables
 * (page_table != NULL) put window slot i of request b at logical position
 * prefix_len[b] + i, resolved through the page table; the byte offset of
 * (page, head h, slot s) is page*stride_page + h*stride_head +
 * s*stride_token.  Dense tables put it at b*stride_batch + i*stride_token
 * + h*stride_head.  All strides are in bytes.
 */
typedef struct {
    uint8_t *base;
    const int32_t *page_table;
    const int32_t *prefix_len;
    int32_t max_pages, page_size;
    int64_t stride_page, stride_token, stride_head, stride_batch;
    int32_t n_heads, row_bytes;
} orc_rows;

static uint8_t *orc_row_addr(const orc_rows *t, int b, int slot, int h)
{
    if (t->page_table) {
        int64_t lp = (int64_t)t->prefix_len[b] + slot;
        int64_t page = t->page_table[(int64_t)b * t->max_pages + lp / t->page_size];
        return t->base + page * t->stride_page + (int64_t)h * t->stride_head +
               (lp % t->page_size) * t->stride_token;
    }
    return t->base + (int64_t)b * t->stride_batch + (int64_t)slot * t->stride_token +
           (int64_t)h * t->stride_head;
}

/*
 * Moves the accepted path to the window's leading slots, in every table:
 * for i < accept_len[b], row i <- row accepted_path[b][i] ([DTS] "The tree
 * is a parameter of the chain path": compact_window_rows copies words, so
 * it does not depend on the dtype; [MEM] "Discarding the rejected branches'
 * KV": slots of the accepted nodes move to the front of the block).  All
 * source rows are read before any row is written; rows from accept_len on,
 * other requests and other bytes are left as they are.
 */
int orc_compact_rows(const orc_rows *tables, int n_tables,
                     const int32_t *accepted_path, const int32_t *accept_len,
                     int B, int N)
{
    for (int ti = 0; ti < n_tables; ++ti) {
        const orc_rows *t = &tables[ti];
        int64_t seg = t->row_bytes;
        uint8_t *snap = (uint8_t *)malloc((size_t)(N * t->n_heads * seg + 1));
        for (int b = 0; b < B; ++b) {
            int a = accept_len[b];
            if (a < 0 || a > N) {
                free(snap);
                return ORC_BAD;
            }
            for (int i = 0; i < a; ++i) {
                int src = accepted_path[(int64_t)b * N + i];
                if (src < 0 || src >= N) {
                    free(snap);
                    return ORC_BAD;
                }
                for (int h = 0; h < t->n_heads; ++h)
                    memcpy(snap + ((int64_t)i * t->n_heads + h) * seg,
                           orc_row_addr(t, b, src, h), (size_t)seg);
            }
            for (int i = 0; i < a; ++i)
                for (int h = 0; h < t->n_heads; ++h)
                    memcpy(orc_row_addr(t, b, i, h),
                           snap + ((int64_t)i * t->n_heads + h) * seg, (size_t)seg);
        }
        free(snap);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* sampled verify: Gumbel-max draws keyed by (seed, position)          */
/* ------------------------------------------------------------------ */

/*
 * Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and
 * Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011): ten rounds
 * of the Philox S-box on a 4 x 32-bit counter under a 2 x 32-bit key.  A
 * round multiplies counter words 0 and 2 by 0xD2511F53 and 0xCD9E8D57 into
 * 64-bit products (hi, lo) and outputs {hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1,
 * lo0}; between rounds the key advances by the Weyl constants 0x9E3779B9
 * and 0xBB67AE85.  The pages name no generator; this one is specified in
 * full by its publication, so the kernels implement it independently.
 */
void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
    }
    for (int i = 0; i < 4; ++i)
        out[i] = c[i];
}

/*
 * The uniform of token v at key position pos under a request seed: Philox
 * counter {v / 4, pos, 0, 0}, key {seed low 32 bits, seed high 32 bits},
 * output word v % 4; its top 24 bits b give u = (b + 1/2) / 2^24 in (0, 1).
 */
double orc_gumbel_uniform(uint64_t seed, int64_t pos, int64_t v)
{
    uint32_t ctr[4] = {(uint32_t)(v / 4), (uint32_t)pos, 0u, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t o[4];
    orc_philox4x32_10(ctr, key, o);
    return ((double)(o[v % 4] >> 8) + 0.5) / 16777216.0;
}

/*
 * Sampled target tokens of every verify row ([DTS] "Sampled verify keys
 * noise by position"): the row of node i of request b draws its token by
 * Gumbel-max, keyed by (seed[b], the position the node predicts), which is
 * positions[b][i] + 1 with positions = vc + depth (so siblings share their
 * noise, and a chain row draws what plain decoding draws at that position).
 *   z_v = logits[v] / T + g_v,   g_v = -ln(-ln u_v),   token = argmax_v z_v
 * with the lowest v winning ties and NaN ranking last (an all-NaN or all
 * -inf row gives token 0).  T = temperature[b]; T <= 0 is greedy: the argmax
 * of the logits themselves.  logits holds dtype elements (0 fp32, 1 bf16),
 * row (b*N + i) at element offset (b*N + i) * row_stride.  zmax (optional)
 * receives the winning z (fp64) and z2 (optional) the best z of any other
 * token, so a caller can tell how close the decision was.
 */
int orc_sample_gumbel(const void *logits, int dtype, int64_t row_stride, int V, int B,
                      int N, const float *temperature, const uint64_t *seed,
                      const int32_t *positions, int32_t *tokens, double *zmax, double *z2)
{
    if (V < 1 || B < 0 || N < 1 || (dtype != 0 && dtype != 1))
        return ORC_BAD;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t row = 0; row < (int64_t)B * N; ++row) {
        int b = (int)(row / N);
        double T = temperature[b];
        int64_t key_pos = (int64_t)positions[row] + 1;
        double best = -INFINITY, second = -INFINITY;
        int arg = 0;
        for (int64_t v = 0; v < V; ++v) {
            double l = orc_load(logits, dtype, row * row_stride + v);
            double z = T > 0 ? l / T - log(-log(orc_gumbel_uniform(seed[b], key_pos, v))) : l;
            if (isnan(z))
                z = -INFINITY;
            if (z > best) {
                second = best;
                best = z;
                arg = (int)v;
            } else if (z > second) {
                second = z;
            }
        }
        tokens[row] = arg;
        if (zmax)
            zmax[row] = best;
        if (z2)
            z2[row] = second;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* tree construction: EAGLE-2 beam, global selection, numbering, links */
/* ------------------------------------------------------------------ */

/* Candidate order of the tree construction: the higher score first, then the
 * lower candidate id; a NaN score ranks after every number ([DTS] "Tree
 * construction is deterministic": equal scores are ordered by candidate id,
 * NaN after all numbers).  Returns 1 when candidate a comes before b. */
static int orc_cand_before(float sa, int a, float sb, int b)
{
    int na = isnan(sa), nb = isnan(sb);
    if (na != nb)
        return nb;           /* the number before the NaN */
    if (!na && sa != sb)
        return sa > sb;
    return a < b;
}

/*
 * One EAGLE-2 expansion step for every request ([MEM] "EAGLE-2: the tree
 * stops being a constant": each surviving path's cumulative score times
 * each child's conditional probability, of which the topk best survive; [ETA] "candidate pool to verify rows": score_list / token_list /
 * parents_list, cumulative path scores).  Survivor s (score scores[b][s],
 * pool index surv_idx[b][s], -1 for the root) has K children with
 * conditional probabilities child_p[b][s][j] and tokens child_tok[b][s][j].
 * Child (s, j) is pool entry pool_base + s*K + j with score
 * scores[b][s] * child_p[b][s][j] (an fp32 product), parent surv_idx[b][s]
 * and its token.  The K best children by orc_cand_before (flat index s*K + j
 * as the id) are the next survivors: next_scores[b][r], next_idx[b][r] =
 * their pool indices, best first.  Pool arrays are [B][C]; 1 <= n_surv,
 * K <= n_surv * K.
 */
int orc_beam_step(const float *scores, const int32_t *surv_idx, const float *child_p,
                  const int32_t *child_tok, int B, int n_surv, int K, int C, int pool_base,
                  float *pool_scores, int32_t *pool_parents, int32_t *pool_tokens,
                  float *next_scores, int32_t *next_idx)
{
    int n = n_surv * K;
    if (B < 0 || n_surv < 1 || K < 1 || pool_base < 0 || pool_base + n > C)
        return ORC_BAD;
    float *cs = (float *)malloc(sizeof(float) * n);
    int *used = (int *)malloc(sizeof(int) * n);
    for (int b = 0; b < B; ++b) {
        for (int s = 0; s < n_surv; ++s)
            for (int j = 0; j < K; ++j) {
                int f = s * K + j;
                float p = child_p[((int64_t)b * n_surv + s) * K + j];
                cs[f] = scores[(int64_t)b * n_surv + s] * p;
                pool_scores[(int64_t)b * C + pool_base + f] = cs[f];
                pool_parents[(int64_t)b * C + pool_base + f] = surv_idx[(int64_t)b * n_surv + s];
                pool_tokens[(int64_t)b * C + pool_base + f] =
                    child_tok[((int64_t)b * n_surv + s) * K + j];
                used[f] = 0;
            }
        /* K times: the best child not taken yet */
        for (int r = 0; r < K; ++r) {
            int best = -1;
            for (int f = 0; f < n; ++f)
                if (!used[f] && (best < 0 || orc_cand_before(cs[f], f, cs[best], best)))
                    best = f;
            used[best] = 1;
            next_scores[(int64_t)b * K + r] = cs[best];
            next_idx[(int64_t)b * K + r] = pool_base + best;
        }
    }
    free(cs);
    free(used);
    return ORC_OK;
}

/*
 * The verify tree of every request from its candidate pool ([MEM]
 * organize_draft_results: flatten the score pool, take the num_draft_token
 * - 1 best, sort the selected indices, gather their tokens, keep the parent
 * topology; [ETA] "the verify root is not an ordinary draft candidate": the
 * previous round's bonus token is prepended as node 0).  Pool entry c of
 * request b has score pool_scores[b][c], parent pool index
 * pool_parents[b][c] (-1 = the root) and token pool_tokens[b][c].
 *
 * The N - 1 best candidates by orc_cand_before are kept.  order 0 numbers
 * them by ascending pool index (the pool order); order 1 numbers the tree
 * in depth-first order, a node's higher-scoring child before its others
 * ([DTS] "Tree construction is deterministic": the top path is then
 * numbered 0, 1, 2, ...).  Node 0 is
 * the root with token root_tokens[b]; parents[b][i] is the node of entry
 * i's parent; selected[b][i] is entry i's pool index (-1 for the root).
 * Every kept candidate's parent must be kept or be the root ([MEM]
 * "Building the mask, for real": a candidate whose parent was dropped is
 * refused or fixed, never promoted to a root),
 * and must precede it in the pool (as every expansion step appends after
 * the candidates it expands);
 * otherwise tree_error[b] = 1 + the first node (in pool order) whose parent
 * is missing, and parents/tokens/selected of b are -1.  C >= N - 1.
 */
int orc_select_candidates(const float *pool_scores, const int32_t *pool_parents,
                          const int32_t *pool_tokens, const int32_t *root_tokens, int B, int C,
                          int N, int order, int32_t *parents, int32_t *tokens,
                          int32_t *selected, int32_t *tree_error)
{
    if (B < 0 || N < 1 || N > 64 || C < N - 1 || (order != 0 && order != 1))
        return ORC_BAD;
    int *kept = (int *)malloc(sizeof(int) * (C + 1));
    int *node_of = (int *)malloc(sizeof(int) * (C + 1));
    for (int b = 0; b < B; ++b) {
        const float *sc = pool_scores + (int64_t)b * C;
        const int32_t *pp = pool_parents + (int64_t)b * C;
        for (int c = 0; c < C; ++c)
            kept[c] = 0;
        /* N - 1 times: the best candidate not taken yet */
        for (int r = 0; r < N - 1; ++r) {
            int best = -1;
            for (int c = 0; c < C; ++c)
                if (!kept[c] && (best < 0 || orc_cand_before(sc[c], c, sc[best], best)))
                    best = c;
            kept[best] = 1;
        }
        /* closure */
        int bad = -1, node = 1;
        for (int c = 0; c < C; ++c) {
            node_of[c] = -1;
            if (!kept[c])
                continue;
            int p = pp[c];
            if (bad < 0 && p != -1 && (p < 0 || p >= c || !kept[p]))
                bad = node;
            node_of[c] = node++;
        }
        if (tree_error)
            tree_error[b] = bad < 0 ? 0 : 1 + bad;
        int32_t *par = parents + (int64_t)b * N, *tok = tokens + (int64_t)b * N;
        int32_t *sel = selected + (int64_t)b * N;
        if (bad >= 0) {
            for (int i = 0; i < N; ++i)
                par[i] = tok[i] = sel[i] = -1;
            continue;
        }
        /* pool order: entry rank among kept candidates by pool index */
        int32_t tmp_sel[64];
        tmp_sel[0] = -1;
        for (int c = 0; c < C; ++c)
            if (kept[c])
                tmp_sel[node_of[c]] = c;
        if (order == 1) {
            /* depth first, best child first: an explicit stack of nodes
             * (pool-order numbers); children pushed worst first */
            int stack[64], sp = 0, next = 0, newnum[64];
            stack[sp++] = 0;
            while (sp > 0) {
                int u = stack[--sp];
                newnum[u] = next++;
                int ch[64], nch = 0;
                for (int i = 1; i < N; ++i) {
                    int pc = pp[tmp_sel[i]];
                    int pu = pc == -1 ? 0 : node_of[pc];
                    if (pu == u)
                        ch[nch++] = i;
                }
                /* sort children best first (insertion sort by the candidate order) */
                for (int x = 1; x < nch; ++x)
                    for (int y = x; y > 0; --y) {
                        int a = ch[y], bb = ch[y - 1];
                        if (orc_cand_before(sc[tmp_sel[a]], tmp_sel[a], sc[tmp_sel[bb]], tmp_sel[bb])) {
                            ch[y] = bb;
                            ch[y - 1] = a;
                        }
                    }
                for (int x = nch - 1; x >= 0; --x)
                    stack[sp++] = ch[x];
            }
            for (int i = 0; i < N; ++i) {
                int c = tmp_sel[i];
                int ni = newnum[i];
                sel[ni] = c;
                if (i == 0) {
                    par[ni] = -1;
                    tok[ni] = root_tokens[b];
                } else {
                    int pc = pp[c];
                    par[ni] = pc == -1 ? 0 : newnum[node_of[pc]];
                    tok[ni] = pool_tokens[(int64_t)b * C + c];
                }
            }
        } else {
            for (int i = 0; i < N; ++i) {
                int c = tmp_sel[i];
                sel[i] = c;
                if (i == 0) {
                    par[i] = -1;
                    tok[i] = root_tokens[b];
                } else {
                    int pc = pp[c];
                    par[i] = pc == -1 ? 0 : node_of[pc];
                    tok[i] = pool_tokens[(int64_t)b * C + c];
                }
            }
        }
    }
    free(kept);
    free(node_of);
    return ORC_OK;
}

/*
 * First-child / next-sibling links of every tree ([MEM] "Flattening, and the
 * two link arrays": retrieve_next_token[p] names the first child of p and
 * retrieve_next_sibling[i] the sibling after i; [DDT] compile_ddtree_retrieve).
 * Children are taken in node order (with depth-first best-child-first
 * numbering, or pool order, that is the order the trees are numbered in);
 * -1 where there is none.
 */
int orc_retrieve_links(const int32_t *parents, int B, int N, int32_t *next_token,
                       int32_t *next_sibling)
{
    if (B < 0 || N < 1)
        return ORC_BAD;
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parents + (int64_t)b * N;
        for (int i = 0; i < N; ++i) {
            next_token[(int64_t)b * N + i] = -1;
            next_sibling[(int64_t)b * N + i] = -1;
            for (int j = 0; j < N; ++j)
                if (par[j] == i) {
                    next_token[(int64_t)b * N + i] = j;
                    break;
                }
            if (par[i] >= 0)
                for (int j = i + 1; j < N; ++j)
                    if (par[j] == par[i]) {
                        next_sibling[(int64_t)b * N + i] = j;
                        break;
                    }
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* MLA: prefix + window + merge, K and V both from one latent row      */
/* ------------------------------------------------------------------ */

/*
 * Tree attention over an MLA latent cache ([DTS] "One tree attention ...",
 * the MLA paragraph).  The cascade is the one of orc_tree_attention; what
 * changes is the key and value: each token stores one latent row, shared by
 * every query head, whose first Dc channels (kv_lora_rank) enter the score
 * against the query's first Dc channels and are also the value, and whose
 * Dr rotary channels after them enter the score against the query's last Dr
 * channels (Dr = 0: no rotary part):
 *   s_t = scale * (sum_{d < Dc} q[d] c_t[d] + sum_{d < Dr} q[Dc + d] r_t[d]),
 *   o = sum_t softmax(s)_t c_t  (Dc channels),  lse2 = base-2 log-sum-exp,
 * over the visible keys of the row: the committed prefix [0, P) and window
 * node j at logical position P + j for the set bits j < W of the row's mask
 * (the same visibility as orc_tree_attention).  The latent row of logical
 * position t is at page_table[b][t / ps] * stride_page + (t % ps) *
 * stride_token, Dc + Dr contiguous elements.  q is [B][R][Hq][Dc + Dr] of
 * dtype qdt (fp32 or bf16), the latent pool of dtype latdt: the same as q,
 * or FP8 E4M3 under a bf16 query.  Under an E4M3 latent cache the absorbed
 * query is an E4M3 value too (the page: the prologue returns it in FP8 and
 * the window kernel widens it back exactly), so every key, prefix and
 * window, is scored with q rounded to E4M3 (orc_e4m3_round).  out is
 * [B][R][Hq][Dc] fp64, lse2 [B][R][Hq]; or n_rows listed rows ((b*R + r)*Hq
 * + h).  sm_scale <= 0 means 1/sqrt(Dc + Dr).
 */
int orc_mla_attention(const void *q, const void *latent, int qdt, int latdt,
                      int64_t stride_page, int64_t stride_token, const int32_t *page_table,
                      int max_pages, int page_size, const int32_t *prefix_len,
                      const uint64_t *masks, int W, int B, int R, int Hq, int Dc, int Dr,
                      double sm_scale, const int64_t *rows, int64_t n_rows, double *out,
                      double *lse2)
{
    if (W < 0 || W > 64 || page_size <= 0 || Dc < 1 || Dr < 0 || (qdt != 0 && qdt != 1) ||
        !(latdt == qdt || (latdt == 2 && qdt == 1)))
        return ORC_BAD;
    const int Dk = Dc + Dr;
    if (sm_scale <= 0.0)
        sm_scale = 1.0 / sqrt((double)Dk);
    int64_t total = rows ? n_rows : (int64_t)B * R * Hq;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t n = 0; n < total; ++n) {
        int64_t id = rows ? rows[n] : n;
        int r = (int)((id / Hq) % R);
        int b = (int)(id / ((int64_t)Hq * R));
        int P = prefix_len[b];
        uint64_t m = masks[(int64_t)b * R + r];
        int nk_max = P + W;
        int64_t *kofs = (int64_t *)malloc(sizeof(int64_t) * (nk_max > 0 ? nk_max : 1));
        double *s = (double *)malloc(sizeof(double) * (nk_max > 0 ? nk_max : 1));
        double *qv = (double *)malloc(sizeof(double) * Dk);
        int nk = 0;
        for (int t = 0; t < P + W; ++t) {
            if (t >= P && !((m >> (t - P)) & 1))
                continue;
            int lp = t / page_size;
            if (lp >= max_pages) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            int64_t page = page_table[(int64_t)b * max_pages + lp];
            kofs[nk++] = page * stride_page + (int64_t)(t % page_size) * stride_token;
        }
        for (int d = 0; d < Dk; ++d) {
            qv[d] = orc_load(q, qdt, id * Dk + d);
            if (latdt == 2)
                qv[d] = orc_e4m3_round(qv[d]);
        }
        double *o = out + n * Dc;
        for (int d = 0; d < Dc; ++d)
            o[d] = 0.0;
        if (nk == 0) {
            lse2[n] = -INFINITY;
        } else {
            double mx = -INFINITY;
            for (int t = 0; t < nk; ++t) {
                double acc = 0.0;
                for (int d = 0; d < Dc; ++d)          /* latent part */
                    acc += qv[d] * orc_load(latent, latdt, kofs[t] + d);
                for (int d = 0; d < Dr; ++d)          /* rotary part */
                    acc += qv[Dc + d] * orc_load(latent, latdt, kofs[t] + Dc + d);
                s[t] = sm_scale * acc;
                if (s[t] > mx)
                    mx = s[t];
            }
            double Z = 0.0;
            for (int t = 0; t < nk; ++t) {
                double w = exp(s[t] - mx);
                Z += w;
                for (int d = 0; d < Dc; ++d)          /* the value is the latent part */
                    o[d] += w * orc_load(latent, latdt, kofs[t] + d);
            }
            for (int d = 0; d < Dc; ++d)
                o[d] /= Z;
            lse2[n] = (mx + log(Z)) / log(2.0);
        }
        free(kofs);
        free(s);
        free(qv);
    }
    return bad ? ORC_BAD : ORC_OK;
}

/* ------------------------------------------------------------------ */
/* sampled verify by tree rejection sampling                           */
/* ------------------------------------------------------------------ */

/* a target weight as the walk uses it: positive finite entries, else 0 */
static double orc_tw(float p)
{
    return (p > 0.0f && p < INFINITY) ? (double)p : 0.0;
}

/*
 * Tree rejection sampling with the draft tokens as fixed candidates
 * ([DDT] "The Implementation": a node's children are tried in descending
 * draft probability and the first one passing the rejection test is
 * accepted; [DTS] "Sampled verify keys noise by position": recursive
 * rejection sampling is exact in distribution).  At node cur the target
 * weights are w(v) = probs[cur][v] (positive finite entries, else 0) with
 * total S; the residual after rejecting tokens R is w restricted to v not in
 * R, of mass S - E with E = sum_{x in R} w(x).  Child c (token x) is
 * accepted with the residual's probability of x:
 *     coin[c] * (S - E) < (x in [0, V) and x not in R ? w(x) : 0)
 * and a rejected valid token joins R.  Children are the nodes c with
 * parents[c] == cur, taken in descending draft_score (all equal when
 * draft_score is NULL), ties to the lower index.  An accepted child
 * continues the walk; otherwise (or once the path holds N nodes) the walk
 * stops at cur and the bonus token is the lowest v whose running sum of the
 * residual exceeds bonus_u[cur] * (its total), summed in v order; the last v
 * of positive residual when rounding leaves none, token 0 when the residual
 * is all zero.  Every candidate token is emitted with its residual
 * probability and the bonus with the rest, so the token emitted at every
 * depth is distributed as the target there.
 * Outputs as orc_verify_greedy: path (-1 padded), accept_len (counts the
 * root), tokens[k] = draft[path[k + 1]] for k + 1 < accept_len and the bonus
 * at k = accept_len - 1, -1 after.  margin (or NULL) gets, per request, the
 * smallest |coin (S - E) - w(x)| / S over its children's tests: how near the
 * walk came to a tie (INFINITY when it tested none).
 */
int orc_verify_rejection(const float *probs, int64_t row_stride, int V,
                         const int32_t *draft, const int32_t *parents,
                         const float *draft_score, const float *coins,
                         const float *bonus_u, int B, int N, int32_t *path,
                         int32_t *accept_len, int32_t *tokens, double *margin)
{
    if (N < 1 || N > 64 || V < 1 || row_stride < V)
        return ORC_BAD;
    for (int b = 0; b < B; ++b) {
        const int32_t *dr = draft + (int64_t)b * N;
        const int32_t *par = parents + (int64_t)b * N;
        int32_t *pb = path + (int64_t)b * N;
        double mg = INFINITY;
        for (int k = 0; k < N; ++k)
            pb[k] = -1;
        int len = 0, cur = 0;
        pb[len++] = cur;
        int32_t rej[64];
        int nrej;
        int bonus = 0;
        for (;;) {
            const float *row = probs + ((int64_t)b * N + cur) * row_stride;
            double S = 0.0;
            for (int v = 0; v < V; ++v)
                S += orc_tw(row[v]);
            double E = 0.0;
            nrej = 0;
            int next = -1;
            if (len < N) {
                int tried[64] = {0};
                for (;;) {
                    /* the untried child of highest draft score, lowest index on ties */
                    int c = -1;
                    for (int j = 0; j < N; ++j) {
                        if (par[j] != cur || tried[j])
                            continue;
                        if (c < 0 || (draft_score && draft_score[(int64_t)b * N + j] >
                                                         draft_score[(int64_t)b * N + c]))
                            c = j;
                    }
                    if (c < 0)
                        break;
                    tried[c] = 1;
                    const int x = dr[c];
                    int valid = x >= 0 && x < V;
                    for (int i = 0; valid && i < nrej; ++i)
                        if (rej[i] == x)
                            valid = 0;
                    const double wx = valid ? orc_tw(row[x]) : 0.0;
                    const double lhs = (double)coins[(int64_t)b * N + c] * (S - E);
                    if (S > 0.0 && fabs(lhs - wx) / S < mg)
                        mg = fabs(lhs - wx) / S;
                    if (lhs < wx) {
                        next = c;
                        break;
                    }
                    if (valid) {
                        E += wx;
                        rej[nrej++] = x;
                    }
                }
            }
            if (next >= 0) {
                cur = next;
                pb[len++] = cur;
                continue;
            }
            /* the bonus draw from the residual at cur */
            double T = 0.0;
            for (int v = 0; v < V; ++v) {
                int out = 0;
                for (int i = 0; i < nrej; ++i)
                    if (rej[i] == v)
                        out = 1;
                T += out ? 0.0 : orc_tw(row[v]);
            }
            bonus = 0;
            if (T > 0.0) {
                const double target = (double)bonus_u[(int64_t)b * N + cur] * T;
                double run = 0.0;
                int last_pos = -1, found = -1;
                for (int v = 0; v < V; ++v) {
                    int out = 0;
                    for (int i = 0; i < nrej; ++i)
                        if (rej[i] == v)
                            out = 1;
                    const double r = out ? 0.0 : orc_tw(row[v]);
                    if (r <= 0.0)
                        continue;
                    last_pos = v;
                    run += r;
                    if (found < 0 && run > target)
                        found = v;
                }
                bonus = found >= 0 ? found : last_pos;
            }
            break;
        }
        accept_len[b] = len;
        if (tokens)
            for (int k = 0; k < N; ++k)
                tokens[(int64_t)b * N + k] =
                    k + 1 < len ? dr[pb[k + 1]] : (k + 1 == len ? bonus : -1);
        if (margin)
            margin[b] = mg;
    }
    return ORC_OK;
}

/*
 * The same walk tested against the draft distribution that drew each node's
 * children ([DTS] "Sampled verify keys noise by position": recursive
 * rejection sampling against the draft q of a node's children, exact in
 * distribution).  At node cur the residual starts as r = w / S (w, S as
 * above) and q = draft_q[cur] (positive finite entries, else 0) over its
 * total Q.  Child c (token x) is accepted when
 *     coin[c] * q(x) / Q < r(x)           (probability min(1, r(x) / q(x)))
 * (x outside [0, V) is rejected); otherwise r becomes max(0, r - q / Q)
 * normalised (all zero when nothing is left).  The bonus is drawn from the
 * final r as above (token 0 when r is all zero).  This is exact when the
 * children are independent draws from q tested in an order that does not
 * depend on the drawn tokens (the multi-candidate speculative sampling
 * argument).  Outputs as orc_verify_rejection; margin covers the tests.
 */
int orc_verify_rejection_q(const float *probs, int64_t row_stride, const float *draft_q,
                           int64_t q_row_stride, int V, const int32_t *draft,
                           const int32_t *parents, const float *draft_score,
                           const float *coins, const float *bonus_u, int B, int N,
                           int32_t *path, int32_t *accept_len, int32_t *tokens, double *margin)
{
    if (N < 1 || N > 64 || V < 1 || row_stride < V || q_row_stride < V)
        return ORC_BAD;
    double *r = malloc(sizeof(double) * (size_t)V);
    if (!r)
        return ORC_BAD;
    for (int b = 0; b < B; ++b) {
        const int32_t *dr = draft + (int64_t)b * N;
        const int32_t *par = parents + (int64_t)b * N;
        int32_t *pb = path + (int64_t)b * N;
        double mg = INFINITY;
        for (int k = 0; k < N; ++k)
            pb[k] = -1;
        int len = 0, cur = 0;
        pb[len++] = cur;
        int bonus = 0;
        for (;;) {
            const float *row = probs + ((int64_t)b * N + cur) * row_stride;
            const float *qrow = draft_q + ((int64_t)b * N + cur) * q_row_stride;
            double S = 0.0, Q = 0.0;
            for (int v = 0; v < V; ++v) {
                S += orc_tw(row[v]);
                Q += orc_tw(qrow[v]);
            }
            for (int v = 0; v < V; ++v)
                r[v] = S > 0.0 ? orc_tw(row[v]) / S : 0.0;
            int next = -1;
            if (len < N) {
                int tried[64] = {0};
                for (;;) {
                    int c = -1;
                    for (int j = 0; j < N; ++j) {
                        if (par[j] != cur || tried[j])
                            continue;
                        if (c < 0 || (draft_score && draft_score[(int64_t)b * N + j] >
                                                         draft_score[(int64_t)b * N + c]))
                            c = j;
                    }
                    if (c < 0)
                        break;
                    tried[c] = 1;
                    const int x = dr[c];
                    if (x >= 0 && x < V) {
                        const double qx = Q > 0.0 ? orc_tw(qrow[x]) / Q : 0.0;
                        const double lhs = (double)coins[(int64_t)b * N + c] * qx;
                        if (fabs(lhs - r[x]) < mg)
                            mg = fabs(lhs - r[x]);
                        if (lhs < r[x]) {
                            next = c;
                            break;
                        }
                    }
                    /* rejected: the residual max(0, r - q) renormalised */
                    double Z = 0.0;
                    for (int v = 0; v < V; ++v) {
                        const double qv = Q > 0.0 ? orc_tw(qrow[v]) / Q : 0.0;
                        r[v] = r[v] > qv ? r[v] - qv : 0.0;
                        Z += r[v];
                    }
                    for (int v = 0; v < V; ++v)
                        r[v] = Z > 0.0 ? r[v] / Z : 0.0;
                }
            }
            if (next >= 0) {
                cur = next;
                pb[len++] = cur;
                continue;
            }
            double T = 0.0;
            for (int v = 0; v < V; ++v)
                T += r[v];
            bonus = 0;
            if (T > 0.0) {
                const double target = (double)bonus_u[(int64_t)b * N + cur] * T;
                double run = 0.0;
                int last_pos = -1, found = -1;
                for (int v = 0; v < V && found < 0; ++v) {
                    if (r[v] <= 0.0)
                        continue;
                    last_pos = v;
                    run += r[v];
                    if (run > target)
                        found = v;
                }
                bonus = found >= 0 ? found : last_pos;
            }
            break;
        }
        accept_len[b] = len;
        if (tokens)
            for (int k = 0; k < N; ++k)
                tokens[(int64_t)b * N + k] =
                    k + 1 < len ? dr[pb[k + 1]] : (k + 1 == len ? bonus : -1);
        if (margin)
            margin[b] = mg;
    }
    free(r);
    return ORC_OK;
}
