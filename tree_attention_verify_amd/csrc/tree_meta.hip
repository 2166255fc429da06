// Tree metadata kernels: ancestor masks, position shifts, the greedy walk
// and the word-copy compaction.  Each request's tree fits one wave64
// (N <= 64), so one lane owns one node and tree-wide steps are ballots and
// shuffles within the wave.
#include <climits>

#include "tav_internal.h"

namespace {

constexpr int kWavesPerBlock = 4;

__device__ inline uint64_t shfl_u64(uint64_t v, int src) {
    uint32_t lo = __shfl((uint32_t)v, src);
    uint32_t hi = __shfl((uint32_t)(v >> 32), src);
    return ((uint64_t)hi << 32) | lo;
}

// Ancestor masks by pointer jumping: lane i keeps acc = the bits of the nodes
// from i up to (not including) its current pointer p, and each round adds the
// segment owned by p and jumps p to p's pointer.  After ceil(log2 N) rounds
// every pointer is the root's -1 and acc holds i and all its ancestors
// ("EAGLE Tree Attention ..." section 1: the visibility rule; "Draft-tree
// speculation", "One tree attention ...": one 64-bit ancestor mask per row).
__global__ void __launch_bounds__(256)
k_build_masks(const int32_t *__restrict__ parents, int B, int N, const int32_t *__restrict__ vc,
              int32_t *__restrict__ depth, uint64_t *__restrict__ masks,
              int32_t *__restrict__ positions, int32_t *__restrict__ tree_error) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (b >= B)
        return;  // uniform per wave
    const bool in = lane < N;
    const int64_t o = (int64_t)b * N + lane;
    const int par = in ? parents[o] : -1;
    // node 0 is the only root; every other parent precedes its child
    // ("Medusa, EAGLE-1/2/3, MTP, and tree attention", "Building the mask,
    // for real": a missing parent is rejected, never treated as a root)
    const bool ok = !in || (lane == 0 ? par == -1 : (par >= 0 && par < lane));
    const uint64_t bad = __ballot(!ok);
    if (bad) {
        if (tree_error && lane == 0)
            tree_error[b] = 1 + (__ffsll((unsigned long long)bad) - 1);
        if (in) {
            masks[o] = 0;
            depth[o] = -1;
            if (positions)
                positions[o] = -1;
        }
        return;
    }
    uint64_t acc = in ? (1ull << lane) : 0ull;
    int p = par;
    while (__ballot(p != -1)) {
        const int src = p < 0 ? lane : p;
        const uint64_t up = shfl_u64(acc, src);
        const int pp = __shfl(p, src);
        if (p != -1) {
            acc |= up;
            p = pp;
        }
    }
    if (in) {
        const int d = __popcll(acc) - 1;
        masks[o] = acc;
        depth[o] = d;
        // "Draft-tree speculation", "Position follows depth, slot follows
        // node index": node i sits at vc + depth[i]
        if (positions)
            positions[o] = (vc ? vc[b] : 0) + d;
    }
    if (tree_error && lane == 0)
        tree_error[b] = 0;
}

// load_step (+1) / compact_rows (-1) shifts ("Draft-tree speculation",
// "Position follows depth, slot follows node index").
__global__ void __launch_bounds__(256)
k_shift_positions(int32_t *__restrict__ pos, const int32_t *__restrict__ depth, int64_t total,
                  int N, int direction) {
    const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (o < total)
        pos[o] += direction * (depth[o] - (int)(o % N));
}

// Greedy walk ("Medusa, EAGLE-1/2/3, MTP, and tree attention", "Walking the
// accepted path"): t = target argmax at the current node; the next node is the
// lowest-index child whose draft token is t; stop when there is none.
__global__ void __launch_bounds__(256)
k_verify_greedy(const int32_t *__restrict__ draft, const int32_t *__restrict__ target,
                const int32_t *__restrict__ parents, int B, int N, int32_t *__restrict__ path,
                int32_t *__restrict__ accept_len, int32_t *__restrict__ tokens) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (b >= B)
        return;
    const bool in = lane < N;
    const int64_t o = (int64_t)b * N + lane;
    const int par = in ? parents[o] : INT_MIN;  // never equals a node index
    const int dr = in ? draft[o] : 0;
    const int tg = in ? target[o] : 0;
    int cur = 0, len = 1;
    int mine = lane == 0 ? 0 : -1;  // lane k holds path[k]
    while (len < N) {
        const int t = __shfl(tg, cur);
        const uint64_t cand = __ballot(in && par == cur && dr == t);
        if (!cand)
            break;
        cur = __ffsll((unsigned long long)cand) - 1;
        if (lane == len)
            mine = cur;
        ++len;
    }
    // tokens emitted along the path: target argmax of each accepted node, the
    // last one being the bonus ("EAGLE Tree Attention ..." section 2)
    const int tok = __shfl(tg, mine < 0 ? 0 : mine);
    if (in) {
        path[o] = mine;
        if (tokens)
            tokens[o] = mine < 0 ? -1 : tok;
    }
    if (lane == 0)
        accept_len[b] = len;
}

// ---------------------------------------------------------------------------
// compaction
// ---------------------------------------------------------------------------

constexpr int kMaxTables = 16;
constexpr int kCompactWords = 256;  // 32-bit words per block and row

struct RowTable {
    char *base;
    const int32_t *page_table;
    const int32_t *prefix_len;
    int64_t num_pages, stride_page, stride_token, stride_head, stride_batch;
    int32_t max_pages, ps_shift, n_heads, row_words, words_per_slot;
};

struct CompactArgs {
    RowTable t[kMaxTables];
    const int32_t *path;
    const int32_t *accept_len;
    int B, N;
};

// Byte address of (request b, window slot, segment h) or nullptr if it falls
// outside the table.
__device__ inline char *row_addr(const RowTable &t, int b, int slot, int h) {
    if (t.page_table) {
        const int64_t lp = (int64_t)t.prefix_len[b] + slot;
        if (lp < 0 || (lp >> t.ps_shift) >= t.max_pages)
            return nullptr;
        const int64_t page = t.page_table[(int64_t)b * t.max_pages + (lp >> t.ps_shift)];
        if (page < 0 || page >= t.num_pages)
            return nullptr;
        return t.base + page * t.stride_page + (int64_t)h * t.stride_head +
               (lp & ((1LL << t.ps_shift) - 1)) * t.stride_token;
    }
    return t.base + (int64_t)b * t.stride_batch + (int64_t)slot * t.stride_token +
           (int64_t)h * t.stride_head;
}

// Block (chunk, b, table): 256 word columns of every accepted row of request
// b.  All sources are read into LDS before any destination is written, so a
// destination that is also a later source (path [0, 2, 5]: slot 2 is read
// for row 1 and written from slot 5) is safe.  Different blocks touch
// disjoint bytes.
__global__ void __launch_bounds__(256) k_compact_rows(CompactArgs a) {
    __shared__ uint32_t stage[64][kCompactWords];
    __shared__ const char *src_row[64];   // segment 0 of the source slot of row i, or null
    __shared__ char *dst_row[64];         // segment 0 of slot i, or null
    const RowTable &t = a.t[blockIdx.z];
    const int b = blockIdx.y;
    const int w = blockIdx.x * kCompactWords + threadIdx.x;
    if (blockIdx.x * kCompactWords >= t.words_per_slot)
        return;  // uniform per block
    int n = a.accept_len[b];
    n = n < 0 ? 0 : (n > a.N ? a.N : n);
    // the row addresses first, all in parallel; then every copy's load is
    // independent of the others
    if ((int)threadIdx.x < n) {
        const int i = threadIdx.x;
        const int src = a.path[(int64_t)b * a.N + i];
        const char *sp = src >= 0 && src < a.N ? row_addr(t, b, src, 0) : nullptr;
        src_row[i] = sp;
        dst_row[i] = sp ? row_addr(t, b, i, 0) : nullptr;
    }
    __syncthreads();
    const bool active = w < t.words_per_slot;
    const int h = active ? w / t.row_words : 0;
    const int64_t off = active ? (int64_t)h * t.stride_head + (int64_t)(w - h * t.row_words) * 4 : 0;
#pragma unroll 8
    for (int i = 0; i < n; ++i) {
        const char *p = src_row[i];
        if (active && p)
            stage[i][threadIdx.x] = *(const uint32_t *)(p + off);
    }
    __syncthreads();
#pragma unroll 8
    for (int i = 0; i < n; ++i) {
        char *p = dst_row[i];
        if (active && p)
            *(uint32_t *)(p + off) = stage[i][threadIdx.x];
    }
}

inline hipStream_t S(void *s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

using tav::Checks;
using tav::str;

extern "C" tav_status tree_build_masks(const int32_t *parents, int32_t B, int32_t N,
                                       const int32_t *vc, int32_t *depth, uint64_t *masks,
                                       int32_t *positions, int32_t *tree_error, void *stream) {
    Checks c;
    TAV_NEED(c, B >= 0, TAV_ERR_INVALID_ARG, "B must be >= 0, got " + str(B));
    TAV_NEED(c, N >= 1 && N <= 64, TAV_ERR_INVALID_ARG, "N must be in [1, 64], got " + str(N));
    if (B > 0) {
        TAV_NEED(c, parents, TAV_ERR_INVALID_ARG, "parents is NULL");
        TAV_NEED(c, depth, TAV_ERR_INVALID_ARG, "depth is NULL");
        TAV_NEED(c, masks, TAV_ERR_INVALID_ARG, "masks is NULL");
    }
    if (c.status != TAV_OK || B == 0)
        return tav::finish("tree_build_masks", c);
    const int blocks = (B + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(k_build_masks, dim3(blocks), dim3(64 * kWavesPerBlock), 0, S(stream),
                       parents, B, N, vc, depth, masks, positions, tree_error);
    return tav::launched("tree_build_masks");
}

extern "C" tav_status tree_shift_positions(int32_t *positions, const int32_t *depth, int32_t B,
                                           int32_t N, int32_t direction, void *stream) {
    Checks c;
    TAV_NEED(c, B >= 0, TAV_ERR_INVALID_ARG, "B must be >= 0, got " + str(B));
    TAV_NEED(c, N >= 1 && N <= 64, TAV_ERR_INVALID_ARG, "N must be in [1, 64], got " + str(N));
    TAV_NEED(c, direction == 1 || direction == -1, TAV_ERR_INVALID_ARG,
             "direction must be +1 or -1, got " + str(direction));
    if (B > 0) {
        TAV_NEED(c, positions, TAV_ERR_INVALID_ARG, "positions is NULL");
        TAV_NEED(c, depth, TAV_ERR_INVALID_ARG, "depth is NULL");
    }
    if (c.status != TAV_OK || B == 0)
        return tav::finish("tree_shift_positions", c);
    const int64_t total = (int64_t)B * N;
    hipLaunchKernelGGL(k_shift_positions, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       S(stream), positions, depth, total, N, direction);
    return tav::launched("tree_shift_positions");
}

extern "C" tav_status verify_tree_greedy(const int32_t *draft_tokens, const int32_t *target_argmax,
                                         const int32_t *parents, int32_t B, int32_t N,
                                         int32_t *accepted_path, int32_t *accept_len,
                                         int32_t *accepted_tokens, void *stream) {
    Checks c;
    TAV_NEED(c, B >= 0, TAV_ERR_INVALID_ARG, "B must be >= 0, got " + str(B));
    TAV_NEED(c, N >= 1 && N <= 64, TAV_ERR_INVALID_ARG, "N must be in [1, 64], got " + str(N));
    if (B > 0) {
        TAV_NEED(c, draft_tokens, TAV_ERR_INVALID_ARG, "draft_tokens is NULL");
        TAV_NEED(c, target_argmax, TAV_ERR_INVALID_ARG, "target_argmax is NULL");
        TAV_NEED(c, parents, TAV_ERR_INVALID_ARG, "parents is NULL");
        TAV_NEED(c, accepted_path, TAV_ERR_INVALID_ARG, "accepted_path is NULL");
        TAV_NEED(c, accept_len, TAV_ERR_INVALID_ARG, "accept_len is NULL");
    }
    if (c.status != TAV_OK || B == 0)
        return tav::finish("verify_tree_greedy", c);
    const int blocks = (B + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(k_verify_greedy, dim3(blocks), dim3(64 * kWavesPerBlock), 0, S(stream),
                       draft_tokens, target_argmax, parents, B, N, accepted_path, accept_len,
                       accepted_tokens);
    return tav::launched("verify_tree_greedy");
}

extern "C" tav_status compact_window_rows(const tav_rows *tables, int32_t n_tables,
                                          const int32_t *accepted_path, const int32_t *accept_len,
                                          int32_t B, int32_t N, void *stream) {
    Checks c;
    TAV_NEED(c, B >= 0, TAV_ERR_INVALID_ARG, "B must be >= 0, got " + str(B));
    TAV_NEED(c, N >= 1 && N <= 64, TAV_ERR_INVALID_ARG, "N must be in [1, 64], got " + str(N));
    TAV_NEED(c, n_tables >= 0, TAV_ERR_INVALID_ARG, "n_tables must be >= 0, got " + str(n_tables));
    TAV_NEED(c, n_tables == 0 || tables, TAV_ERR_INVALID_ARG, "tables is NULL");
    if (B > 0 && n_tables > 0) {
        TAV_NEED(c, accepted_path, TAV_ERR_INVALID_ARG, "accepted_path is NULL");
        TAV_NEED(c, accept_len, TAV_ERR_INVALID_ARG, "accept_len is NULL");
    }
    for (int i = 0; tables && i < n_tables; ++i) {
        const tav_rows &t = tables[i];
        const std::string p = "tables[" + str(i) + "].";
        TAV_NEED(c, t.base, TAV_ERR_INVALID_ARG, p + "base is NULL");
        TAV_NEED(c, ((uintptr_t)t.base & 3) == 0, TAV_ERR_INVALID_ARG,
                 p + "base is not 4-byte aligned");
        TAV_NEED(c, t.n_heads >= 1, TAV_ERR_INVALID_ARG, p + "n_heads must be >= 1");
        TAV_NEED(c, t.row_bytes > 0 && t.row_bytes % 4 == 0, TAV_ERR_INVALID_ARG,
                 p + "row_bytes must be a positive multiple of 4, got " + str(t.row_bytes));
        TAV_NEED(c, (long long)t.n_heads * (t.row_bytes / 4) <= (1LL << 30), TAV_ERR_INVALID_ARG,
                 p + "n_heads * row_bytes is too large");
        TAV_NEED(c, t.stride_token % 4 == 0 && t.stride_head % 4 == 0 && t.stride_page % 4 == 0 &&
                     t.stride_batch % 4 == 0,
                 TAV_ERR_INVALID_ARG, p + "strides must be multiples of 4 bytes");
        if (t.page_table) {
            TAV_NEED(c, t.prefix_len, TAV_ERR_INVALID_ARG,
                     p + "prefix_len is NULL for a paged table");
            TAV_NEED(c, t.max_pages >= 1, TAV_ERR_INVALID_ARG, p + "max_pages must be >= 1");
            TAV_NEED(c, tav::is_pow2(t.page_size) && t.page_size <= 1024, TAV_ERR_INVALID_ARG,
                     p + "page_size must be a power of two in [1, 1024], got " + str(t.page_size));
            TAV_NEED(c, t.num_pages >= 1, TAV_ERR_INVALID_ARG, p + "num_pages must be >= 1");
        }
    }
    if (c.status != TAV_OK || B == 0 || n_tables == 0)
        return tav::finish("compact_window_rows", c);
    for (int first = 0; first < n_tables; first += kMaxTables) {
        const int n = n_tables - first < kMaxTables ? n_tables - first : kMaxTables;
        CompactArgs a{};
        int max_words = 0;
        for (int i = 0; i < n; ++i) {
            const tav_rows &s = tables[first + i];
            RowTable &t = a.t[i];
            t.base = (char *)s.base;
            t.page_table = s.page_table;
            t.prefix_len = s.prefix_len;
            t.num_pages = s.num_pages;
            t.stride_page = s.stride_page;
            t.stride_token = s.stride_token;
            t.stride_head = s.stride_head;
            t.stride_batch = s.stride_batch;
            t.max_pages = s.max_pages;
            t.ps_shift = s.page_table ? tav::ilog2(s.page_size) : 0;
            t.n_heads = s.n_heads;
            t.row_words = s.row_bytes / 4;
            t.words_per_slot = s.n_heads * t.row_words;
            if (t.words_per_slot > max_words)
                max_words = t.words_per_slot;
        }
        a.path = accepted_path;
        a.accept_len = accept_len;
        a.B = B;
        a.N = N;
        const unsigned chunks = (unsigned)((max_words + kCompactWords - 1) / kCompactWords);
        hipLaunchKernelGGL(k_compact_rows, dim3(chunks, (unsigned)B, (unsigned)n), dim3(256), 0,
                           S(stream), a);
        tav_status st = tav::launched("compact_window_rows");
        if (st != TAV_OK)
            return st;
    }
    return TAV_OK;
}
