// Tree construction: the step before the verify path.
//
//   k_beam_step        one EAGLE-2 expansion: the survivors' cumulative scores
//                      times the new conditional probabilities (fp32), the
//                      pool entries of the step, and the topk best paths
//                      ("Medusa, EAGLE-1/2/3, MTP, and tree attention",
//                      "EAGLE-2: the tree stops being a constant").
//   k_select_tree      the N - 1 best candidates of a request's pool, the
//                      previous bonus token prepended as node 0, numbered in
//                      pool order or depth first, a node's higher-scoring
//                      child before its others; closure is checked ("Draft-tree speculation",
//                      "Tree construction is deterministic"; the course
//                      chapter's organize_draft_results; "a missing parent is
//                      rejected, never treated as a root").
//   k_retrieve_links   first-child / next-sibling arrays (the course chapter,
//                      "Flattening, and the two link arrays").
//
// Candidate order everywhere: the higher score first, the lower candidate id
// on equal scores, NaN after every number.  One workgroup per request: the
// pools are a few hundred to a few thousand candidates and the trees at most
// 64 nodes, so each request's work is a handful of LDS passes and wave
// ballots; these kernels are latency-bound.
#include <climits>
#include <cmath>

#include "tav_internal.h"

namespace {

constexpr int kBuildThreads = 256;
constexpr int kSelectThreads = 1024;    // the rank phase of the selection
constexpr int kMaxBeamCands = 1024;     // n_surv * K per step
constexpr int kMaxPool = 8192;          // candidates per request

// Lane j's value in every lane (j wave-uniform): v_readlane, no LDS trip.
__device__ inline int lane_val(int x, int j) { return __builtin_amdgcn_readlane(x, j); }
__device__ inline uint64_t lane_val(uint64_t x, int j) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(x >> 32), j) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, j);
}

// The candidate order as integers: a key that increases with the score
// (equal for -0 and +0, the lowest for NaN), then the lower id first.
__device__ inline int order_key(float s) {
    s = s + 0.0f;                         // -0 -> +0
    const int i = __float_as_int(s);
    const int k = i >= 0 ? i : (i ^ 0x7fffffff);
    return s != s ? INT_MIN : k;
}
__device__ inline bool before_k(int ka, int a, int kb, int b) {
    return ka > kb || (ka == kb && a < b);
}

// Rank of candidate (z, id) in an LDS array of n scores: how many come
// before it, counted up to `limit` (the count may pass it by up to 7).  The
// scan goes 8 entries per check of the limit, so the LDS reads (the same
// address in every lane: broadcasts) are issued back to back.
__device__ inline int rank_in(const int *key, int n, int kz, int id, int limit) {
    int rank = 0, g = 0;
    for (; g + 8 <= n && rank < limit; g += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
            rank += before_k(key[g + u], g + u, kz, id) ? 1 : 0;
    }
    for (; g < n && rank < limit; ++g)
        rank += before_k(key[g], g, kz, id) ? 1 : 0;
    return rank;
}

__global__ void __launch_bounds__(kBuildThreads)
k_beam_step(const float *__restrict__ scores, const int32_t *__restrict__ surv_idx,
            const float *__restrict__ child_p, const int32_t *__restrict__ child_tok, int n_surv,
            int K, int C, int pool_base, float *__restrict__ pool_scores,
            int32_t *__restrict__ pool_parents, int32_t *__restrict__ pool_tokens,
            float *next_scores, int32_t *next_idx) {
    __shared__ float cs[kMaxBeamCands];
    __shared__ int ck[kMaxBeamCands];
    const int b = blockIdx.x;
    const int n = n_surv * K;
    // every input is read before any output is written (the survivor arrays
    // may be updated in place)
    int32_t par_of[kMaxBeamCands / kBuildThreads];
    for (int f = threadIdx.x, k = 0; f < n; f += kBuildThreads, ++k) {
        const int s = f / K;
        cs[f] = scores[(int64_t)b * n_surv + s] * child_p[(int64_t)b * n + f];
        ck[f] = order_key(cs[f]);
        par_of[k] = surv_idx[(int64_t)b * n_surv + s];
    }
    __syncthreads();
    for (int f = threadIdx.x, k = 0; f < n; f += kBuildThreads, ++k) {
        const float z = cs[f];
        pool_scores[(int64_t)b * C + pool_base + f] = z;
        pool_parents[(int64_t)b * C + pool_base + f] = par_of[k];
        pool_tokens[(int64_t)b * C + pool_base + f] = child_tok[(int64_t)b * n + f];
        const int rank = rank_in(ck, n, ck[f], f, K);
        if (rank < K) {
            next_scores[(int64_t)b * K + rank] = z;
            next_idx[(int64_t)b * K + rank] = pool_base + f;
        }
    }
}

// One workgroup per request.  Phase 1 ranks every candidate against the pool
// (stopping at N - 1 better ones) and records the kept ones by rank; phase 2
// (wave 0, lane = node) orders them, links parents, checks closure and, for
// the depth-first numbering, computes each node's preorder index from its
// ancestor mask and its better siblings' subtree sizes.
__global__ void __launch_bounds__(kSelectThreads)
k_select_tree(const float *__restrict__ pool_scores, const int32_t *__restrict__ pool_parents,
              const int32_t *__restrict__ pool_tokens, const int32_t *__restrict__ root_tokens,
              int C, int N, int order, int32_t *__restrict__ parents, int32_t *__restrict__ tokens,
              int32_t *__restrict__ selected, int32_t *__restrict__ tree_error) {
    __shared__ int sk[kMaxPool];
    __shared__ int32_t spar[kMaxPool];
    __shared__ int32_t stok[kMaxPool];
    __shared__ int32_t kept[64];
    const int b = blockIdx.x;
    const float *ps = pool_scores + (int64_t)b * C;
    // the whole pool is staged in LDS with coalesced loads, so the per-node
    // steps below read no global memory
    for (int c = threadIdx.x; c < C; c += kSelectThreads) {
        sk[c] = order_key(ps[c]);
        spar[c] = pool_parents[(int64_t)b * C + c];
        stok[c] = pool_tokens[(int64_t)b * C + c];
    }
    __syncthreads();
    const int M = N - 1;
    for (int c = threadIdx.x; c < C; c += kSelectThreads) {
        const int rank = rank_in(sk, C, sk[c], c, M);
        if (rank < M)
            kept[rank] = c;
    }
    __syncthreads();
    // node numbers in pool order: node 0 is the root, kept entry c is
    // 1 + (number of kept entries with a lower pool index); wave 0 works on,
    // lane = node, and every later step stays inside that wave
    __shared__ int32_t cand_of[64];
    const int lane = threadIdx.x;
    const bool in = lane < N;
    if (in) {
        const int c = lane >= 1 ? kept[lane - 1] : -1;       // kept by rank
        int node = 0;
        if (lane >= 1) {
            for (int j = 0; j < M; ++j)
                node += kept[j] < c ? 1 : 0;
            node += 1;
        }
        cand_of[node] = c;
    }
    __syncthreads();
    if (threadIdx.x >= 64)
        return;
    // lane i now takes pool-order node i
    const int ci = in ? cand_of[lane] : -1;
    const int p0 = (in && lane >= 1) ? spar[ci] : -1;
    int pn = p0 == -1 ? 0 : -1;
    for (int j = 1; j < N; ++j) {
        const int cj = lane_val(ci, j);
        pn = (p0 >= 0 && cj == p0) ? j : pn;
    }
    const bool bad = in && lane >= 1 && (p0 < -1 || p0 >= ci || pn < 0);
    pn = (in && lane >= 1) ? pn : -1;
    const uint64_t badm = __ballot(bad);
    int32_t *par = parents + (int64_t)b * N, *tok = tokens + (int64_t)b * N;
    int32_t *sel = selected + (int64_t)b * N;
    if (badm) {
        if (lane == 0 && tree_error)
            tree_error[b] = 1 + (__ffsll((unsigned long long)badm) - 1);
        if (in)
            par[lane] = tok[lane] = sel[lane] = -1;
        return;
    }
    if (lane == 0 && tree_error)
        tree_error[b] = 0;
    const int my_tok = !in ? 0 : (lane == 0 ? root_tokens[b] : stok[ci]);
    if (order == 0) {
        if (in) {
            par[lane] = lane == 0 ? -1 : pn;
            tok[lane] = my_tok;
            sel[lane] = ci;
        }
        return;
    }
    // depth first, best child first.  Ancestor masks by pointer jumping
    // (pool-order parents precede their children).
    uint64_t acc = in ? (1ull << lane) : 0ull;
    int p = in ? (lane == 0 ? -1 : pn) : -1;
    while (__ballot(p != -1)) {
        const int src = p < 0 ? lane : p;
        const uint32_t ulo = __shfl((uint32_t)acc, src), uhi = __shfl((uint32_t)(acc >> 32), src);
        const int pp = __shfl(p, src);
        if (p != -1) {
            acc |= ((uint64_t)uhi << 32) | ulo;
            p = pp;
        }
    }
    // subtree sizes: how many nodes have this one among their ancestors
    int size = 0;
    for (int j = 0; j < N; ++j)
        size += (int)((lane_val(acc, j) >> lane) & 1);
    // offset within the parent's block: 1 + the sizes of the better siblings
    const int my_k = (in && lane >= 1) ? sk[ci] : 0;
    int offset = 1;
    for (int j = 1; j < N; ++j) {
        const int pj = lane_val(pn, j);
        const int cj = lane_val(ci, j);
        const int kj = lane_val(my_k, j);
        const int szj = lane_val(size, j);
        offset += (in && lane >= 1 && j != lane && pj == pn && before_k(kj, cj, my_k, ci)) ? szj : 0;
    }
    // preorder index: the offsets of the node and its ancestors (root 0)
    int pre = 0;
    for (int j = 1; j < N; ++j) {
        const int oj = lane_val(offset, j);
        if ((acc >> j) & 1)
            pre += oj;
    }
    const int par_pre = __shfl(pre, pn < 0 ? 0 : pn);
    if (in) {
        par[pre] = lane == 0 ? -1 : par_pre;
        tok[pre] = my_tok;
        sel[pre] = ci;
    }
}

// First child and next sibling in node order; one wave per request.
__global__ void __launch_bounds__(256)
k_retrieve_links(const int32_t *__restrict__ parents, int B, int N, int32_t *__restrict__ next_token,
                 int32_t *__restrict__ next_sibling) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (b >= B)
        return;
    const bool in = lane < N;
    const int par = in ? parents[(int64_t)b * N + lane] : INT_MIN;
    int nt = -1;
    for (int i = 0; i < N; ++i) {
        const uint64_t m = __ballot(in && par == i);
        if (lane == i && m)
            nt = __ffsll((unsigned long long)m) - 1;
    }
    // next sibling: the lowest later lane with the same parent
    int ns = -1;
    for (int j = N - 1; j >= 1; --j) {
        const int pj = lane_val(par, j);
        ns = (in && j > lane && pj == par && par >= 0) ? j : ns;
    }
    if (in) {
        next_token[(int64_t)b * N + lane] = nt;
        next_sibling[(int64_t)b * N + lane] = ns;
    }
}

inline hipStream_t S(void *s) { return (hipStream_t)s; }

}  // namespace

using tav::Checks;
using tav::str;

extern "C" tav_status tree_beam_step(const float *scores, const int32_t *surv_idx,
                                     const float *child_p, const int32_t *child_tok, int32_t B,
                                     int32_t n_surv, int32_t K, int32_t C, int32_t pool_base,
                                     float *pool_scores, int32_t *pool_parents,
                                     int32_t *pool_tokens, float *next_scores, int32_t *next_idx,
                                     void *stream) {
    Checks c;
    TAV_NEED(c, B >= 0, TAV_ERR_INVALID_ARG, "B must be >= 0, got " + str(B));
    TAV_NEED(c, n_surv >= 1 && K >= 1, TAV_ERR_INVALID_ARG,
             "n_surv and K must be >= 1, got " + str(n_surv) + ", " + str(K));
    TAV_NEED(c, (long long)n_surv * K <= kMaxBeamCands, TAV_ERR_UNSUPPORTED,
             "n_surv * K must be <= " + str(kMaxBeamCands) + ", got " + str((long long)n_surv * K));
    TAV_NEED(c, pool_base >= 0 && (long long)pool_base + (long long)n_surv * K <= C,
             TAV_ERR_INVALID_ARG,
             "pool entries [pool_base, pool_base + n_surv * K) must lie in [0, C)");
    if (B > 0) {
        TAV_NEED(c, scores && surv_idx && child_p && child_tok, TAV_ERR_INVALID_ARG,
                 "scores, surv_idx, child_p and child_tok must be set");
        TAV_NEED(c, pool_scores && pool_parents && pool_tokens, TAV_ERR_INVALID_ARG,
                 "pool_scores, pool_parents and pool_tokens must be set");
        TAV_NEED(c, next_scores && next_idx, TAV_ERR_INVALID_ARG,
                 "next_scores and next_idx must be set");
    }
    if (c.status != TAV_OK || B == 0)
        return tav::finish("tree_beam_step", c);
    hipLaunchKernelGGL(k_beam_step, dim3((unsigned)B), dim3(kBuildThreads), 0, S(stream), scores,
                       surv_idx, child_p, child_tok, n_surv, K, C, pool_base, pool_scores,
                       pool_parents, pool_tokens, next_scores, next_idx);
    return tav::launched("tree_beam_step");
}

extern "C" tav_status tree_select_candidates(const float *pool_scores, const int32_t *pool_parents,
                                             const int32_t *pool_tokens,
                                             const int32_t *root_tokens, int32_t B, int32_t C,
                                             int32_t N, int32_t order, int32_t *parents,
                                             int32_t *tokens, int32_t *selected,
                                             int32_t *tree_error, void *stream) {
    Checks c;
    TAV_NEED(c, B >= 0, TAV_ERR_INVALID_ARG, "B must be >= 0, got " + str(B));
    TAV_NEED(c, N >= 1 && N <= 64, TAV_ERR_INVALID_ARG, "N must be in [1, 64], got " + str(N));
    TAV_NEED(c, C >= N - 1 && C >= 1, TAV_ERR_INVALID_ARG,
             "C must be >= max(1, N - 1), got " + str(C));
    TAV_NEED(c, C <= kMaxPool, TAV_ERR_UNSUPPORTED,
             "C must be <= " + str(kMaxPool) + ", got " + str(C));
    TAV_NEED(c, order == 0 || order == 1, TAV_ERR_INVALID_ARG,
             "order must be 0 (pool order) or 1 (depth first), got " + str(order));
    if (B > 0) {
        TAV_NEED(c, pool_scores && pool_parents && pool_tokens && root_tokens, TAV_ERR_INVALID_ARG,
                 "pool_scores, pool_parents, pool_tokens and root_tokens must be set");
        TAV_NEED(c, parents && tokens && selected, TAV_ERR_INVALID_ARG,
                 "parents, tokens and selected must be set");
    }
    if (c.status != TAV_OK || B == 0)
        return tav::finish("tree_select_candidates", c);
    hipLaunchKernelGGL(k_select_tree, dim3((unsigned)B), dim3(kSelectThreads), 0, S(stream),
                       pool_scores, pool_parents, pool_tokens, root_tokens, C, N, order, parents,
                       tokens, selected, tree_error);
    return tav::launched("tree_select_candidates");
}

extern "C" tav_status tree_retrieve_links(const int32_t *parents, int32_t B, int32_t N,
                                          int32_t *next_token, int32_t *next_sibling,
                                          void *stream) {
    Checks c;
    TAV_NEED(c, B >= 0, TAV_ERR_INVALID_ARG, "B must be >= 0, got " + str(B));
    TAV_NEED(c, N >= 1 && N <= 64, TAV_ERR_INVALID_ARG, "N must be in [1, 64], got " + str(N));
    if (B > 0)
        TAV_NEED(c, parents && next_token && next_sibling, TAV_ERR_INVALID_ARG,
                 "parents, next_token and next_sibling must be set");
    if (c.status != TAV_OK || B == 0)
        return tav::finish("tree_retrieve_links", c);
    hipLaunchKernelGGL(k_retrieve_links, dim3((unsigned)((B + 3) / 4)), dim3(256), 0, S(stream),
                       parents, B, N, next_token, next_sibling);
    return tav::launched("tree_retrieve_links");
}
