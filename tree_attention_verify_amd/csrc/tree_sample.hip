// Sampled verify, two ways:
//   - Gumbel-max target draws of every verify row, keyed by (request seed,
//     the position the node predicts), walked by verify_tree_greedy;
//   - tree rejection sampling of the draft tokens against the target rows
//     (k_verify_rejection<false>, and k_verify_rejection<true> against the
//     draft distribution that drew each node's children), further below.
//
// "Draft-tree speculation", section "Sampled verify keys noise by position":
// each verify row's target token is a Gumbel-max draw whose noise is
// indexed by the request's seed and a position, for a tree the position the
// node predicts (vc + depth + 1) rather than its row; acceptance is then the greedy tree walk
// over the draws (verify_tree_greedy with the draws as the target tokens).
//
// Noise: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011) with counter
// {v / 4, key position, 0, 0} and key {seed low, seed high}; output word
// v % 4 of token v gives u = (top 24 bits + 1/2) / 2^24 and
// g = -ln(-ln u).  z_v = logit_v / T + g_v; the token is the argmax, the
// lowest index winning ties, NaN ranking last; T <= 0 takes the argmax of
// the logits.
//
// The logits of a row are streamed once (HBM-bound at small work per
// element, vector-ALU bound at the ~30 instructions per element of the
// noise): grid = (rows, vocabulary chunks), 256 threads, each thread taking
// 8 consecutive tokens per step (one 16-byte load for bf16, two for fp32,
// two Philox blocks).  Each chunk writes its best (z, token) to the
// workspace; one wave per row then reduces the chunks.
#include <climits>
#include <cmath>

#include "tav_internal.h"

namespace {

constexpr int kSampleThreads = 256;
constexpr int kSampleMaxChunks = 64;
constexpr int kSampleMinChunk = 4096;   // tokens per chunk at least

struct Philox4 {
    uint32_t w[4];
};

// Ten rounds of the Philox4x32 S-box: words 0 and 2 are multiplied by the
// round multipliers into 64-bit products; the high halves are mixed with
// words 1 and 3 and the round key, the low halves pass on; the key advances
// by the Weyl increments between rounds.
__device__ inline Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                        uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return {{c0, c1, c2, c3}};
}

constexpr float kLn2 = 0.69314718055994531f;

// g = -ln(-ln u) for u = (b + 1/2) / 2^24, b the top 24 bits of a Philox
// word.  E = -ln u: for u > 1 - 2^-7 the series w + w^2/2 + w^3/3 + w^4/4 in
// w = 1 - u = (2^24 - 1 - b + 1/2) / 2^24, which is exact in fp32 there
// (relative error of the series < w^4 / 5); else the hardware log2 of u
// (u itself is rounded to fp32 there, an error below 2^-25).  Then g = -ln E.
// Both forms are computed and one is selected, so the loop has no branch.
__device__ inline float gumbel_of(uint32_t word) {
    const uint32_t bits = word >> 8;
    const float u = ((float)bits + 0.5f) * (1.f / 16777216.f);
    const float w = ((float)(16777215u - bits) + 0.5f) * (1.f / 16777216.f);
    const float es = w * (1.f + w * (0.5f + w * (1.f / 3.f + w * 0.25f)));
    const float el = -__builtin_amdgcn_logf(u) * kLn2;
    return -__builtin_amdgcn_logf(w < 0.0078125f ? es : el) * kLn2;
}

// (z, v) ordering: larger z first, then the lower token.  NaN never gets
// here (it is mapped to -inf).
__device__ inline bool better(float z, int v, float bz, int bv) {
    return z > bz || (z == bz && v < bv);
}

struct SampleArgs {
    const void *logits;
    int64_t row_stride;
    int V, N, chunk, n_chunks;
    const float *temperature;
    const uint64_t *seed;
    const int32_t *positions;
    float *part_z;
    int32_t *part_v;
    int32_t *tokens;
};

template <bool BF16>
__global__ void __launch_bounds__(kSampleThreads) k_gumbel_partial(SampleArgs a) {
    const int row = blockIdx.x;
    const int b = row / a.N;
    const float T = a.temperature[b];
    const bool noise = T > 0.f;
    const float invT = noise ? 1.f / T : 1.f;
    const uint64_t sd = a.seed[b];
    const uint32_t k0 = (uint32_t)sd, k1 = (uint32_t)(sd >> 32);
    const uint32_t kpos = (uint32_t)(a.positions[row] + 1);
    const int lo = blockIdx.y * a.chunk;
    const int hi = min(a.V, lo + a.chunk);

    // Each thread scans increasing tokens, so a strict comparison keeps the
    // lowest token among equal scores; starting from the thread's first
    // token makes a run of -inf scores give that token.  fmaxf(z, -inf)
    // maps NaN to -inf.
    float bz = -INFINITY;
    int bv = lo + 8 * (int)threadIdx.x < hi ? lo + 8 * (int)threadIdx.x : INT_MAX;
    auto visit = [&](float l, int v, uint32_t word) {
        const float z = fmaxf(noise ? fmaf(l, invT, gumbel_of(word)) : l, -INFINITY);
        const bool t = z > bz;
        bz = t ? z : bz;
        bv = t ? v : bv;
    };
    for (int v0 = lo + 8 * threadIdx.x; v0 < hi; v0 += 8 * kSampleThreads) {
        float l[8];
        if (v0 + 8 <= hi) {
            if constexpr (BF16) {
                const int4 x = *(const int4 *)((const uint16_t *)a.logits + row * a.row_stride + v0);
                const uint32_t u32[4] = {(uint32_t)x.x, (uint32_t)x.y, (uint32_t)x.z, (uint32_t)x.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    l[2 * e] = __uint_as_float(u32[e] << 16);
                    l[2 * e + 1] = __uint_as_float(u32[e] & 0xffff0000u);
                }
            } else {
                const float4 x0 = *(const float4 *)((const float *)a.logits + row * a.row_stride + v0);
                const float4 x1 = *(const float4 *)((const float *)a.logits + row * a.row_stride + v0 + 4);
                l[0] = x0.x; l[1] = x0.y; l[2] = x0.z; l[3] = x0.w;
                l[4] = x1.x; l[5] = x1.y; l[6] = x1.z; l[7] = x1.w;
            }
        } else {
            // past the chunk end: -inf, which never replaces the best
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int v = v0 + e < hi ? v0 + e : hi - 1;
                if constexpr (BF16)
                    l[e] = __uint_as_float((uint32_t)((const uint16_t *)a.logits)[row * a.row_stride + v] << 16);
                else
                    l[e] = ((const float *)a.logits)[row * a.row_stride + v];
                l[e] = v0 + e < hi ? l[e] : -INFINITY;
            }
        }
        Philox4 r0{}, r1{};
        if (noise) {
            r0 = philox4x32_10((uint32_t)(v0 >> 2), kpos, 0u, 0u, k0, k1);
            r1 = philox4x32_10((uint32_t)(v0 >> 2) + 1u, kpos, 0u, 0u, k0, k1);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
            visit(l[e], v0 + e, e < 4 ? r0.w[e] : r1.w[e - 4]);
    }

    // workgroup reduction of (bz, bv)
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float z2 = __shfl_xor(bz, o);
        const int v2 = __shfl_xor(bv, o);
        if (better(z2, v2, bz, bv)) {
            bz = z2;
            bv = v2;
        }
    }
    __shared__ float sz[kSampleThreads / 64];
    __shared__ int sv[kSampleThreads / 64];
    const int wv = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        sz[wv] = bz;
        sv[wv] = bv;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < kSampleThreads / 64; ++i)
            if (better(sz[i], sv[i], bz, bv)) {
                bz = sz[i];
                bv = sv[i];
            }
        a.part_z[(int64_t)row * a.n_chunks + blockIdx.y] = bz;
        a.part_v[(int64_t)row * a.n_chunks + blockIdx.y] = bv;
    }
}

// One wave per row: the best of its chunks.  A row whose every z is -inf
// (all logits -inf or NaN) gets token 0, the lowest index among equal maxima.
__global__ void __launch_bounds__(256) k_gumbel_reduce(SampleArgs a, int rows) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows)
        return;
    float bz = -INFINITY;
    int bv = INT_MAX;
    if (lane < a.n_chunks) {
        bz = a.part_z[(int64_t)row * a.n_chunks + lane];
        bv = a.part_v[(int64_t)row * a.n_chunks + lane];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float z2 = __shfl_xor(bz, o);
        const int v2 = __shfl_xor(bv, o);
        if (better(z2, v2, bz, bv)) {
            bz = z2;
            bv = v2;
        }
    }
    if (lane == 0)
        a.tokens[row] = bv;
}

struct SamplePlan {
    int chunk, n_chunks;
    size_t z_bytes, bytes;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

SamplePlan sample_plan(int B, int N, int V) {
    SamplePlan p{};
    const long long rows = (long long)B * N;
    int n = rows > 0 ? (int)((2048 + rows - 1) / rows) : 1;   // >= 2048 workgroups
    const int by_size = (V + kSampleMinChunk - 1) / kSampleMinChunk;
    n = n < by_size ? n : by_size;
    n = n < kSampleMaxChunks ? n : kSampleMaxChunks;
    n = n < 1 ? 1 : n;
    int chunk = (V + n - 1) / n;
    chunk = (chunk + 7) / 8 * 8;      // chunks start on 8-token (Philox block pair) boundaries
    p.chunk = chunk;
    p.n_chunks = (V + chunk - 1) / chunk;
    p.z_bytes = align256((size_t)rows * p.n_chunks * sizeof(float));
    p.bytes = p.z_bytes + align256((size_t)rows * p.n_chunks * sizeof(int32_t));
    return p;
}

// ---------------------------------------------------------------------------
// Tree rejection sampling ("From Greedy to Sampling ...", section "The
// Implementation": a node's children are tried in descending draft
// probability and the first passing the rejection test is accepted;
// "Draft-tree speculation", section "Sampled verify keys noise by position":
// recursive rejection sampling is exact in distribution).
//
// Fixed candidates (no draft q): child c of node cur (token x) is accepted
// when coin[c] * (S - E) < w(x), with w the node's target row (positive
// finite entries, else 0), S its total and E the weight of the distinct
// tokens already rejected there, which leave the residual; the walk ends
// with a bonus token drawn from the residual by inverse CDF.
// Against the drafter's q for the children: at node cur r_0 = w / S and
// q^ = q / Q (positive finite entries); child i (token x) in the trying
// order is accepted when coin * q^(x) < r_i(x), else r_{i+1} = max(0, r_i -
// q^) / Z_{i+1}.  r_i(v) depends only on w(v), q(v), S, Q and Z_1 .. Z_i, so
// a test reads two floats and each rejection costs one pass over the node's
// two rows for the next Z; the bonus draws from the final residual.
//
// Work split.  One workgroup streams a row at about the bandwidth of one CU,
// so every pass over a node's rows is cut into slices of 64 tiles of 256
// tokens and shared by the G workgroups of the request.  The G members all
// walk the tree: each computes its slices of a pass (member m takes slices
// m, m + G, ...), stores each slice's total as one 64-bit word {total, pass
// tag}, and reads every slice's word back until all carry the pass's tag;
// they then hold the same totals and take the same decisions, so no
// workgroup has to announce one.  The slice results depend only on the
// slice, and the totals are summed in slice order, so the outcome does not
// depend on which workgroup computed what.  Requests are dealt to
// workgroups in the order they start (a ticket counter in the workspace),
// G consecutive tickets per request: only the last request to be dealt can
// be waiting for a member that has not started, and every earlier request
// runs to its end and frees its CUs, so the grid needs no more than G
// workgroups resident at once.  Every wait polls at most kRejSpin times; a
// request whose wait gives up (which a working device never makes happen)
// reports accept_len -1.
//
// Slice passes: each wave sums four tiles (lane l holds tokens 4 l .. 4 l +
// 3 of a tile, 16-byte loads, tokens past V count 0) by butterflies side by
// side, then wave 0 reduces the slice's 64 tile sums: by an inclusive scan
// for the passes the bonus draw reads (the tile sums go to the workspace),
// by a butterfly for the other totals.  Slot words alternate between two
// sets by pass parity: a member starts pass P + 2 only after every member
// has stored pass P + 1, which each does only after reading pass P.
//
// Bonus (member 0): the tile sums of the final node's residual (for fixed
// candidates the last row pass's, with the tiles of rejected tokens summed
// again without them) are rescanned per slice; the slice totals are walked
// in order to the slice where the running sum passes u * total, then that
// slice's running tile sums to the tile, then the tile's lanes (four tokens
// each) to the token; where fp32 rounding leaves no crossing at a level, the
// last positive entry of that level is taken.
constexpr int kRejWaves = 16;
constexpr int kRejThreads = 64 * kRejWaves;
constexpr int kRejTile = 256;                          // tokens per tile: 64 lanes x 4
constexpr int kRejSlice = 64;                          // tiles per slice
constexpr int kRejWaveTiles = kRejSlice / kRejWaves;   // tiles per wave and slice
constexpr int kRejMaxV = 1 << 20;
constexpr int kRejMaxTiles = kRejMaxV / kRejTile;
constexpr int kRejMaxSlices = kRejMaxTiles / kRejSlice;
constexpr int kRejSpin = 1 << 20;                      // polls before a wait gives up
constexpr int kRejTargetGroups = 256;                  // workgroups aimed for: one per CU

enum : int {
    kPassRowP = 1,     // tile sums of w (fixed candidates)
    kPassRowPQ = 2,    // totals of w and of q
    kPassZ = 3,        // total of max(r_k - q^, 0)
    kPassBonusQ = 4,   // tile sums of r_k
};

// One per request in the workspace, cleared before every call.
struct RejCtl {
    uint64_t tot[2][kRejMaxSlices];    // per slice {total (fp32 bits), tag}, by pass parity
    uint64_t tot2[2][kRejMaxSlices];   // the second total of a pass (of q), likewise
};

struct RejArgs {
    const float *probs;
    int64_t row_stride;
    const float *q;                    // the draft q rows, or NULL
    int64_t q_row_stride;
    int32_t V, N, B, G, nslices;
    const int32_t *draft, *parents;
    const float *score, *coins, *bonus_u;
    int32_t *path, *accept_len, *tokens;
    int *ticket;
    RejCtl *ctl;                       // [B]
    float *tsum;                       // [B][2][nslices * 64] tile sums, by pass parity
};

__device__ inline float rej_w(float p) { return (p > 0.f && p < INFINITY) ? p : 0.f; }

// sum over the 64 lanes; every lane gets the same value (the butterfly adds
// the same two operands on both partners)
__device__ inline float rej_wave_sum(float x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
        x += __shfl_xor(x, m, 64);
    return x;
}

// inclusive prefix sum over the 64 lanes
__device__ inline float rej_wave_scan(float x, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float y = __shfl_up(x, d, 64);
        if (lane >= d)
            x += y;
    }
    return x;
}

__device__ inline float lane_f(float v, int i) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), i));
}

// the residual after k rejections against q at a token with entries p, q
__device__ inline float rej_resid(float pv, float qv, int k, float iS, float iQ,
                                  const float *zinv) {
    float r = rej_w(pv) * iS;
    const float qh = rej_w(qv) * iQ;
    for (int j = 0; j < k; ++j)
        r = fmaxf(r - qh, 0.f) * zinv[j];
    return r;
}

__device__ inline uint64_t rej_word(float v, uint32_t tag) {
    return ((uint64_t)tag << 32) | __float_as_uint(v);
}

// Wave 0: lane g < nslices gets slice g's total (and second total when
// `two`) of the pass tagged `tag`, polling each slot at agent scope
// (acquire) until it carries the tag; false if the wait gave up.
__device__ inline bool rej_wait_totals(RejCtl *ctl, int par, uint32_t tag, int nslices, bool two,
                                       int lane, float &x, float &y) {
    bool have = lane >= nslices, have2 = !two || lane >= nslices;
    x = 0.f;
    y = 0.f;
    for (int it = 0; it < kRejSpin; ++it) {
        if (!have) {
            const uint64_t v =
                __hip_atomic_load(&ctl->tot[par][lane], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
            if ((uint32_t)(v >> 32) == tag) {
                have = true;
                x = __uint_as_float((uint32_t)v);
            }
        }
        if (!have2) {
            const uint64_t v =
                __hip_atomic_load(&ctl->tot2[par][lane], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
            if ((uint32_t)(v >> 32) == tag) {
                have2 = true;
                y = __uint_as_float((uint32_t)v);
            }
        }
        if (__ballot(!(have && have2)) == 0)
            return true;
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

// The term of one token in a pass.
template <int KIND>
__device__ inline float rej_term(float pv, float qv, int k, float iS, float iQ, const float *zinv) {
    if constexpr (KIND == kPassRowP || KIND == kPassRowPQ)
        return rej_w(pv);
    else if constexpr (KIND == kPassZ)
        return fmaxf(rej_resid(pv, qv, k, iS, iQ, zinv) - rej_w(qv) * iQ, 0.f);
    else
        return rej_resid(pv, qv, k, iS, iQ, zinv);
}

// Slice s of pass `tag` (parity par) over the rows of node `node` of
// request b: every thread takes part; wave 0 stores the results (the tile
// sums and then, with release order, the slice's tagged total).
template <int KIND>
__device__ __attribute__((always_inline)) void rej_slice(
    const RejArgs &a, int b, int node, int k, float iS, float iQ, const float *zinv, int s,
    int par, uint32_t tag, float *lt, float *lt2, int lane, int w) {
    constexpr bool LQ = KIND != kPassRowP;   // the q row too
    const int V = a.V;
    const int nfull = V / kRejTile;
    const int ntiles = (V + kRejTile - 1) / kRejTile;
    const int64_t ri = (int64_t)b * a.N + node;
    const float *row = a.probs + ri * a.row_stride;
    const float *qrow = LQ ? a.q + ri * a.q_row_stride : nullptr;
    const int t0 = s * kRejSlice + w * kRejWaveTiles;
    float4 pv[kRejWaveTiles], qv[kRejWaveTiles];
#pragma unroll
    for (int i = 0; i < kRejWaveTiles; ++i) {
        const int t = t0 + i;   // wave-uniform
        pv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        qv[i] = pv[i];
        if (t < nfull) {
            pv[i] = *(const float4 *)(row + (int64_t)t * kRejTile + lane * 4);
            if constexpr (LQ)
                qv[i] = *(const float4 *)(qrow + (int64_t)t * kRejTile + lane * 4);
        } else if (t < ntiles) {
            const int v0 = t * kRejTile + lane * 4;
            pv[i].x = v0 < V ? row[v0] : 0.f;
            pv[i].y = v0 + 1 < V ? row[v0 + 1] : 0.f;
            pv[i].z = v0 + 2 < V ? row[v0 + 2] : 0.f;
            pv[i].w = v0 + 3 < V ? row[v0 + 3] : 0.f;
            if constexpr (LQ) {
                qv[i].x = v0 < V ? qrow[v0] : 0.f;
                qv[i].y = v0 + 1 < V ? qrow[v0 + 1] : 0.f;
                qv[i].z = v0 + 2 < V ? qrow[v0 + 2] : 0.f;
                qv[i].w = v0 + 3 < V ? qrow[v0 + 3] : 0.f;
            }
        }
    }
    float x[kRejWaveTiles], y[kRejWaveTiles];
#pragma unroll
    for (int i = 0; i < kRejWaveTiles; ++i) {
        auto f = [&](float p, float q) { return rej_term<KIND>(p, q, k, iS, iQ, zinv); };
        x[i] = (f(pv[i].x, qv[i].x) + f(pv[i].y, qv[i].y)) +
               (f(pv[i].z, qv[i].z) + f(pv[i].w, qv[i].w));
        y[i] = KIND == kPassRowPQ ? (rej_w(qv[i].x) + rej_w(qv[i].y)) +
                                        (rej_w(qv[i].z) + rej_w(qv[i].w))
                                  : 0.f;
    }
    // the tiles' butterflies side by side (the same sums as rej_wave_sum)
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
#pragma unroll
        for (int i = 0; i < kRejWaveTiles; ++i) {
            x[i] += __shfl_xor(x[i], m, 64);
            if constexpr (KIND == kPassRowPQ)
                y[i] += __shfl_xor(y[i], m, 64);
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < kRejWaveTiles; ++i) {
            lt[w * kRejWaveTiles + i] = x[i];
            lt2[w * kRejWaveTiles + i] = y[i];
        }
    }
    __syncthreads();
    if (w == 0) {
        RejCtl *ctl = a.ctl + b;
        if constexpr (KIND == kPassRowP || KIND == kPassBonusQ) {
            const float xv = lt[lane];
            const float inc = rej_wave_scan(xv, lane);
            const int ntp = a.nslices * kRejSlice;
            a.tsum[((int64_t)b * 2 + par) * ntp + s * kRejSlice + lane] = xv;
            if (lane == 63)   // after the wave's tile sums (release)
                __hip_atomic_store(&ctl->tot[par][s], rej_word(inc, tag), __ATOMIC_RELEASE,
                                   __HIP_MEMORY_SCOPE_AGENT);
        } else {
            const float sx = rej_wave_sum(lt[lane]);
            const float sy = rej_wave_sum(lt2[lane]);
            if (lane == 0) {
                if constexpr (KIND == kPassRowPQ)
                    __hip_atomic_store(&ctl->tot2[par][s], rej_word(sy, tag), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&ctl->tot[par][s], rej_word(sx, tag), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    __syncthreads();   // lt is free again
}

template <class R>
__device__ __attribute__((always_inline)) int rej_bonus_draw(
    const float *tsum, float *tinc, float *gs, int nslices, int V, float u, R r, int lane,
    int w) {
    for (int g = w; g < nslices; g += kRejWaves) {
        const float inc = rej_wave_scan(tsum[g * kRejSlice + lane], lane);
        tinc[g * kRejSlice + lane] = inc;
        if (lane == 63)
            gs[g] = inc;
    }
    __syncthreads();
    int bonus = 0;
    if (w == 0) {
        float total = 0.f;
        for (int g = 0; g < nslices; ++g)
            total += gs[g];
        const float target = u * total;
        int g = -1, lastg = -1;
        float before = 0.f, run = 0.f;
        for (int i = 0; i < nslices; ++i) {
            const float x = gs[i];
            if (x > 0.f) {
                lastg = i;
                if (g < 0 && run + x > target) {
                    g = i;
                    before = run;
                }
            }
            run += x;
        }
        if (total > 0.f) {
            bool crossed = g >= 0;
            if (!crossed)
                g = lastg;
            const float x = tsum[g * kRejSlice + lane];
            const float inc = tinc[g * kRejSlice + lane];
            const uint64_t hit = __ballot(crossed && x > 0.f && before + inc > target);
            const uint64_t nz = __ballot(x > 0.f);
            int l;
            if (hit) {
                l = __builtin_ctzll(hit);
            } else {
                crossed = false;
                l = nz ? 63 - __builtin_clzll(nz) : 0;
            }
            const float bt = before + (l > 0 ? tinc[g * kRejSlice + l - 1] : 0.f);
            const int k = g * kRejSlice + l;
            // tile k: lane m holds its tokens 4 m .. 4 m + 3; the first lane
            // whose running sum passes the target scans its four
            const int v0 = k * kRejTile + lane * 4;
            float rr[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                rr[e] = v0 + e < V ? r(v0 + e) : 0.f;
            const float ls = ((rr[0] + rr[1]) + rr[2]) + rr[3];
            const float inc2 = rej_wave_scan(ls, lane);
            const float up = __shfl_up(inc2, 1, 64);
            const float exc2 = lane > 0 ? up : 0.f;
            const uint64_t hit2 = __ballot(crossed && ls > 0.f && bt + inc2 > target);
            const uint64_t nz2 = __ballot(ls > 0.f);
            const int l2 = hit2 ? __builtin_ctzll(hit2) : (nz2 ? 63 - __builtin_clzll(nz2) : 0);
            int e_pick = -1, e_last = -1;
            float cum = bt + exc2;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (rr[e] > 0.f) {
                    e_last = e;
                    cum += rr[e];
                    if (hit2 && e_pick < 0 && cum > target)
                        e_pick = e;
                }
            }
            const int e_sel = e_pick >= 0 ? e_pick : e_last;
            bonus = k * kRejTile + 4 * l2 + __shfl(e_sel < 0 ? 0 : e_sel, l2, 64);
        }
    }
    return bonus;
}

__global__ void k_rej_clear(uint4 *p, int64_t n16) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

template <bool WQ>
__global__ void __launch_bounds__(kRejThreads) k_verify_rejection(RejArgs a) {
    __shared__ float lt[kRejSlice], lt2[kRejSlice];
    __shared__ float tsum[kRejMaxTiles];          // member 0: the bonus tile sums
    __shared__ float tinc[kRejMaxTiles];          // member 0: their running sums per slice
    __shared__ float gs[kRejMaxSlices];
    __shared__ float s_zinv[64];
    __shared__ int32_t s_par[64], s_dr[64], s_path[64], s_rej[64], s_ord[64];
    __shared__ float s_sc[64], s_coin[64], s_bu[64], s_px[64], s_qx[64];
    __shared__ int s_ticket, s_fail, s_next, s_nrej, s_nk, s_acc, s_bonus;
    __shared__ float s_S, s_Q;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (tid == 0)
        s_ticket = atomicAdd(a.ticket, 1);
    __syncthreads();
    const int b = s_ticket / a.G, mem = s_ticket % a.G;
    RejCtl *ctl = a.ctl + b;
    const int N = a.N, V = a.V;
    const int64_t nb = (int64_t)b * N;
    if (tid < N) {
        s_par[tid] = a.parents[nb + tid];
        s_dr[tid] = a.draft[nb + tid];
        s_sc[tid] = a.score ? a.score[nb + tid] : 0.f;
        s_coin[tid] = a.coins[nb + tid];
        s_bu[tid] = a.bonus_u[nb + tid];
    }
    if (tid == 0) {
        s_path[0] = 0;
        s_fail = 0;
    }
    __syncthreads();

    int P = 0;   // passes so far; pass P has tag P + 1 and parity P & 1
    // this member's slices of pass P
    auto pass = [&](int kind, int node, int k, float iS, float iQ) __attribute__((always_inline)) {
        const int par = P & 1;
        const uint32_t tag = (uint32_t)P + 1;
        for (int s = mem; s < a.nslices; s += a.G) {
            if (kind == kPassRowP)
                rej_slice<kPassRowP>(a, b, node, k, iS, iQ, s_zinv, s, par, tag, lt, lt2, lane, w);
            else if (kind == kPassRowPQ)
                rej_slice<kPassRowPQ>(a, b, node, k, iS, iQ, s_zinv, s, par, tag, lt, lt2, lane, w);
            else if (kind == kPassZ)
                rej_slice<kPassZ>(a, b, node, k, iS, iQ, s_zinv, s, par, tag, lt, lt2, lane, w);
            else
                rej_slice<kPassBonusQ>(a, b, node, k, iS, iQ, s_zinv, s, par, tag, lt, lt2, lane,
                                       w);
        }
    };

    int cur = 0, len = 1, nrej = 0;
    float iS = 0.f, iQ = 0.f;
    bool ok = true;
    for (;;) {
        const float *row = a.probs + (nb + cur) * a.row_stride;
        if constexpr (!WQ) {
            // wave 0, lane j = node j: a child's token weight, loaded before
            // the pass so that its latency overlaps it
            const bool is_child = w == 0 && lane < N && len < N && s_par[lane] == cur;
            const int xj = lane < N ? s_dr[lane] : -1;
            const bool valid = is_child && xj >= 0 && xj < V;
            const float wx = valid ? rej_w(row[xj]) : 0.f;
            pass(kPassRowP, cur, 0, 0.f, 0.f);
            if (w == 0) {
                // Siblings are tried in descending draft score, the lower
                // index on ties: child j's rank counts the children before
                // it, E_j the weight of the distinct valid tokens before it
                // (all rejected if the walk reaches j), and a token repeating
                // an earlier sibling's has no residual weight.
                const float scj = lane < N ? s_sc[lane] : 0.f;
                const uint64_t cm = __ballot(is_child), vmask = __ballot(valid);
                int rank = 0;
                bool dup = false;
                for (uint64_t m = cm; m; m &= m - 1) {   // the children only, i wave-uniform
                    const int i = __builtin_ctzll(m);
                    const float sci = lane_f(scj, i);
                    const int xi = __builtin_amdgcn_readlane(xj, i);
                    const bool before = sci > scj || (sci == scj && i < lane);
                    rank += before ? 1 : 0;
                    dup = dup || (before && ((vmask >> i) & 1) && xi == xj);
                }
                const uint64_t fmask = __ballot(valid && !dup);
                float Ej = 0.f;
                for (uint64_t m = cm; m; m &= m - 1) {
                    const int i = __builtin_ctzll(m);
                    const float sci = lane_f(scj, i);
                    const float wi = lane_f(wx, i);
                    const bool before = sci > scj || (sci == scj && i < lane);
                    Ej += (before && ((fmask >> i) & 1)) ? wi : 0.f;
                }
                const float wxe = valid && !dup ? wx : 0.f;
                // the row total: the slice totals in slice order
                float gx, unused;
                if (!rej_wait_totals(ctl, P & 1, (uint32_t)P + 1, a.nslices, false, lane, gx,
                                     unused)) {
                    if (lane == 0) {
                        s_fail = 1;
                        s_next = -1;
                    }
                } else {
                    float S = 0.f;
                    for (int g = 0; g < a.nslices; ++g)
                        S += lane_f(gx, g);
                    const bool pass_ = is_child && s_coin[lane < N ? lane : 0] * (S - Ej) < wxe;
                    // the first passing child in the trying order
                    int best = pass_ ? rank : 64;
#pragma unroll
                    for (int m = 1; m < 64; m <<= 1)
                        best = min(best, __shfl_xor(best, m, 64));
                    const uint64_t win = __ballot(pass_ && rank == best);
                    const int next = win ? __builtin_ctzll(win) : -1;
                    // tokens rejected at this node when the walk stops here:
                    // every valid child token
                    const uint64_t vm = __ballot(valid);
                    if (valid)
                        s_rej[__builtin_popcountll(vm & ((1ull << lane) - 1))] = xj;
                    if (lane == 0) {
                        s_next = next;
                        s_nrej = next >= 0 ? 0 : __builtin_popcountll(vm);
                    }
                }
            }
            __syncthreads();
            ++P;
            if (s_fail) {
                ok = false;
                break;
            }
        } else {
            const float *qrow = a.q + (nb + cur) * a.q_row_stride;
            // the children in their trying order, and their tokens' entries
            // of both rows, loaded before the pass
            if (w == 0) {
                const bool is_child = lane < N && len < N && s_par[lane] == cur;
                const int xj = lane < N ? s_dr[lane] : -1;
                const bool valid = is_child && xj >= 0 && xj < V;
                const float scj = lane < N ? s_sc[lane] : 0.f;
                const uint64_t cm = __ballot(is_child);
                int rank = 0;
                for (uint64_t m = cm; m; m &= m - 1) {
                    const int i = __builtin_ctzll(m);
                    const float sci = lane_f(scj, i);
                    rank += (sci > scj || (sci == scj && i < lane)) ? 1 : 0;
                }
                if (is_child)
                    s_ord[rank] = lane;
                if (lane < N) {
                    s_px[lane] = valid ? row[xj] : 0.f;
                    s_qx[lane] = valid ? qrow[xj] : 0.f;
                }
                if (lane == 0)
                    s_nk = __builtin_popcountll(cm);
            }
            pass(kPassRowPQ, cur, 0, 0.f, 0.f);
            if (w == 0) {
                float sx, sy;
                if (!rej_wait_totals(ctl, P & 1, (uint32_t)P + 1, a.nslices, true, lane, sx, sy)) {
                    if (lane == 0)
                        s_fail = 1;
                } else {
                    float S = 0.f, Q = 0.f;
                    for (int g = 0; g < a.nslices; ++g) {
                        S += lane_f(sx, g);
                        Q += lane_f(sy, g);
                    }
                    if (lane == 0) {
                        s_S = S;
                        s_Q = Q;
                    }
                }
            }
            __syncthreads();
            ++P;
            if (s_fail) {
                ok = false;
                break;
            }
            iS = s_S > 0.f ? 1.f / s_S : 0.f;
            iQ = s_Q > 0.f ? 1.f / s_Q : 0.f;
            const int nk = s_nk;
            int next = -1;
            nrej = 0;
            for (int i = 0; i < nk; ++i) {
                const int c = s_ord[i];
                if (tid == 0) {
                    const int x = s_dr[c];
                    bool acc = false;
                    if (x >= 0 && x < V)
                        acc = s_coin[c] * (rej_w(s_qx[c]) * iQ) <
                              rej_resid(s_px[c], s_qx[c], i, iS, iQ, s_zinv);
                    s_acc = acc;
                }
                __syncthreads();
                if (s_acc) {
                    next = c;
                    break;
                }
                // rejected: Z_{i+1} = sum_v max(0, r_i(v) - q^(v))
                pass(kPassZ, cur, i, iS, iQ);
                if (w == 0) {
                    float sx, unused;
                    if (!rej_wait_totals(ctl, P & 1, (uint32_t)P + 1, a.nslices, false, lane, sx,
                                         unused)) {
                        if (lane == 0)
                            s_fail = 1;
                    } else {
                        float z = 0.f;
                        for (int g = 0; g < a.nslices; ++g)
                            z += lane_f(sx, g);
                        if (lane == 0)
                            s_zinv[i] = z > 0.f ? 1.f / z : 0.f;
                    }
                }
                __syncthreads();
                ++P;
                if (s_fail) {
                    ok = false;
                    break;
                }
                nrej = i + 1;
            }
            if (!ok)
                break;
            if (tid == 0)
                s_next = next;
            __syncthreads();
        }
        const int next = s_next;
        if (next < 0)
            break;
        if (tid == 0)
            s_path[len] = next;
        cur = next;
        ++len;
        __syncthreads();
    }
    if constexpr (WQ) {
        if (ok)
            pass(kPassBonusQ, cur, nrej, iS, iQ);
    }
    if (mem != 0)
        return;   // member 0 draws the bonus and writes the results
    if constexpr (WQ) {
        if (ok) {
            if (w == 0) {
                float sx, unused;
                if (!rej_wait_totals(ctl, P & 1, (uint32_t)P + 1, a.nslices, false, lane, sx,
                                     unused) &&
                    lane == 0)
                    s_fail = 1;
            }
            __syncthreads();
            ++P;
            ok = s_fail == 0;
        }
    }
    if (!ok) {
        if (tid < N) {
            a.path[nb + tid] = -1;
            if (a.tokens)
                a.tokens[nb + tid] = -1;
        }
        if (tid == 0)
            a.accept_len[b] = -1;
        return;
    }

    // the bonus from the tile sums of the last tile pass (its slots were read
    // with acquire order above)
    const int ntp = a.nslices * kRejSlice;
    const float *ts = a.tsum + ((int64_t)b * 2 + ((P - 1) & 1)) * ntp;
    for (int i = tid; i < ntp; i += kRejThreads)
        tsum[i] = ts[i];
    const float *row = a.probs + (nb + cur) * a.row_stride;
    int bonus;
    if constexpr (!WQ) {
        __syncthreads();
        // the tiles holding rejected tokens summed again without them
        const int nr = s_nrej;
        for (int i = w; i < nr; i += kRejWaves) {
            const int t = s_rej[i] / kRejTile;
            const int v0 = t * kRejTile + lane * 4;
            float r[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int v = v0 + e;
                r[e] = v < V ? rej_w(row[v]) : 0.f;
                for (int k = 0; k < nr; ++k)
                    r[e] = s_rej[k] == v ? 0.f : r[e];
            }
            const float s = rej_wave_sum((r[0] + r[1]) + (r[2] + r[3]));
            if (lane == 0)
                tsum[t] = s;   // waves sharing a tile write the same value
        }
        __syncthreads();
        bonus = rej_bonus_draw(tsum, tinc, gs, a.nslices, V, s_bu[cur],
                               [&](int v) {
                                   float x = rej_w(row[v]);
                                   for (int k = 0; k < nr; ++k)
                                       x = s_rej[k] == v ? 0.f : x;
                                   return x;
                               },
                               lane, w);
    } else {
        __syncthreads();
        const float *qrow = a.q + (nb + cur) * a.q_row_stride;
        const int k = nrej;
        bonus = rej_bonus_draw(tsum, tinc, gs, a.nslices, V, s_bu[cur],
                               [&](int v) { return rej_resid(row[v], qrow[v], k, iS, iQ, s_zinv); },
                               lane, w);
    }
    if (tid == 0)
        s_bonus = bonus;
    __syncthreads();
    if (tid < N) {
        a.path[nb + tid] = tid < len ? s_path[tid] : -1;
        if (a.tokens)
            a.tokens[nb + tid] = tid + 1 < len ? s_dr[s_path[tid + 1]] : (tid + 1 == len ? s_bonus : -1);
    }
    if (tid == 0)
        a.accept_len[b] = len;
}

struct RejPlan {
    int nslices, G;
    size_t zero_bytes, ctl_off, tsum_off, bytes;
};

RejPlan rej_plan(int B, int V) {
    RejPlan p{};
    const int ntiles = (V + kRejTile - 1) / kRejTile;
    p.nslices = (ntiles + kRejSlice - 1) / kRejSlice;
    int G = B > 0 ? (kRejTargetGroups + B - 1) / B : 1;
    G = G < p.nslices ? G : p.nslices;
    p.G = G < 1 ? 1 : G;
    p.ctl_off = 256;
    p.zero_bytes = p.ctl_off + align256((size_t)B * sizeof(RejCtl));
    p.tsum_off = p.zero_bytes;
    p.bytes = p.tsum_off + align256((size_t)B * 2 * p.nslices * kRejSlice * sizeof(float));
    return p;
}

inline hipStream_t S(void *s) { return (hipStream_t)s; }

}  // namespace

using tav::Checks;
using tav::str;

extern "C" size_t tree_sample_workspace_size(int32_t B, int32_t N, int32_t V) {
    if (B < 0 || N < 1 || V < 1)
        return 0;
    return sample_plan(B, N, V).bytes;
}

extern "C" tav_status tree_sample_gumbel(const void *logits, tav_dtype dtype, int64_t row_stride,
                                         int32_t V, int32_t B, int32_t N, const float *temperature,
                                         const uint64_t *seed, const int32_t *positions,
                                         int32_t *tokens, void *workspace, size_t workspace_bytes,
                                         void *stream) {
    Checks c;
    TAV_NEED(c, B >= 0, TAV_ERR_INVALID_ARG, "B must be >= 0, got " + str(B));
    TAV_NEED(c, N >= 1 && N <= 64, TAV_ERR_INVALID_ARG, "N must be in [1, 64], got " + str(N));
    TAV_NEED(c, V >= 1, TAV_ERR_INVALID_ARG, "V must be >= 1, got " + str(V));
    TAV_NEED(c, dtype == TAV_BF16 || dtype == TAV_F32, TAV_ERR_UNSUPPORTED,
             "logits dtype must be TAV_BF16 or TAV_F32, got " + str(dtype));
    const int elem = dtype == TAV_F32 ? 4 : 2;
    TAV_NEED(c, row_stride >= V, TAV_ERR_INVALID_ARG,
             "row_stride must be >= V, got " + str(row_stride) + " < " + str(V));
    TAV_NEED(c, (row_stride * elem) % 16 == 0, TAV_ERR_INVALID_ARG,
             "row_stride must span a multiple of 16 bytes, got " + str(row_stride) + " elements");
    TAV_NEED(c, (long long)B * N * row_stride < (1LL << 62), TAV_ERR_INVALID_ARG,
             "logits too large");
    if (B > 0) {
        TAV_NEED(c, logits, TAV_ERR_INVALID_ARG, "logits is NULL");
        TAV_NEED(c, ((uintptr_t)logits & 15) == 0, TAV_ERR_INVALID_ARG,
                 "logits is not 16-byte aligned");
        TAV_NEED(c, temperature, TAV_ERR_INVALID_ARG, "temperature is NULL");
        TAV_NEED(c, seed, TAV_ERR_INVALID_ARG, "seed is NULL");
        TAV_NEED(c, positions, TAV_ERR_INVALID_ARG, "positions is NULL");
        TAV_NEED(c, tokens, TAV_ERR_INVALID_ARG, "tokens is NULL");
        if (c.status == TAV_OK) {
            const SamplePlan p = sample_plan(B, N, V);
            TAV_NEED(c, workspace, TAV_ERR_WORKSPACE, "workspace is NULL");
            TAV_NEED(c, ((uintptr_t)workspace & 255) == 0, TAV_ERR_WORKSPACE,
                     "workspace is not 256-byte aligned");
            TAV_NEED(c, workspace_bytes >= p.bytes, TAV_ERR_WORKSPACE,
                     "workspace too small: " + str((long long)workspace_bytes) + " < " +
                         str((long long)p.bytes) + " bytes");
        }
    }
    if (c.status != TAV_OK || B == 0)
        return tav::finish("tree_sample_gumbel", c);
    const SamplePlan p = sample_plan(B, N, V);
    SampleArgs a{};
    a.logits = logits;
    a.row_stride = row_stride;
    a.V = V;
    a.N = N;
    a.chunk = p.chunk;
    a.n_chunks = p.n_chunks;
    a.temperature = temperature;
    a.seed = seed;
    a.positions = positions;
    a.part_z = (float *)workspace;
    a.part_v = (int32_t *)((char *)workspace + p.z_bytes);
    a.tokens = tokens;
    const int rows = B * N;
    const dim3 grid((unsigned)rows, (unsigned)p.n_chunks);
    if (dtype == TAV_BF16)
        hipLaunchKernelGGL(k_gumbel_partial<true>, grid, dim3(kSampleThreads), 0, S(stream), a);
    else
        hipLaunchKernelGGL(k_gumbel_partial<false>, grid, dim3(kSampleThreads), 0, S(stream), a);
    tav_status st = tav::launched("tree_sample_gumbel");
    if (st != TAV_OK)
        return st;
    hipLaunchKernelGGL(k_gumbel_reduce, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, S(stream),
                       a, rows);
    return tav::launched("tree_sample_gumbel");
}

extern "C" size_t verify_tree_rejection_workspace_size(int32_t B, int32_t N, int32_t V) {
    if (B < 0 || N < 1 || N > 64 || V < 1 || V > kRejMaxV)
        return 0;
    return rej_plan(B, V).bytes;
}

extern "C" tav_status verify_tree_rejection(const float *probs, int64_t row_stride, int32_t V,
                                            const float *draft_q, int64_t q_row_stride,
                                            const int32_t *draft_tokens, const int32_t *parents,
                                            const float *draft_score, const float *coins,
                                            const float *bonus_u, int32_t B, int32_t N,
                                            int32_t *accepted_path, int32_t *accept_len,
                                            int32_t *accepted_tokens, void *workspace,
                                            size_t workspace_bytes, void *stream) {
    Checks c;
    TAV_NEED(c, B >= 0, TAV_ERR_INVALID_ARG, "B must be >= 0, got " + str(B));
    TAV_NEED(c, N >= 1 && N <= 64, TAV_ERR_INVALID_ARG, "N must be in [1, 64], got " + str(N));
    TAV_NEED(c, V >= 1 && V <= kRejMaxV, TAV_ERR_INVALID_ARG,
             "V must be in [1, " + str(kRejMaxV) + "], got " + str(V));
    TAV_NEED(c, row_stride >= V, TAV_ERR_INVALID_ARG,
             "row_stride must be >= V, got " + str(row_stride) + " < " + str(V));
    TAV_NEED(c, row_stride % 4 == 0, TAV_ERR_INVALID_ARG,
             "row_stride must be a multiple of 4 elements, got " + str(row_stride));
    TAV_NEED(c, (long long)B * N * row_stride < (1LL << 62), TAV_ERR_INVALID_ARG,
             "probs too large");
    if (draft_q) {
        TAV_NEED(c, q_row_stride >= V, TAV_ERR_INVALID_ARG,
                 "q_row_stride must be >= V, got " + str(q_row_stride) + " < " + str(V));
        TAV_NEED(c, q_row_stride % 4 == 0, TAV_ERR_INVALID_ARG,
                 "q_row_stride must be a multiple of 4 elements, got " + str(q_row_stride));
        TAV_NEED(c, ((uintptr_t)draft_q & 15) == 0, TAV_ERR_INVALID_ARG,
                 "draft_q is not 16-byte aligned");
        TAV_NEED(c, (long long)B * N * q_row_stride < (1LL << 62), TAV_ERR_INVALID_ARG,
                 "draft_q too large");
    }
    if (B > 0) {
        TAV_NEED(c, probs, TAV_ERR_INVALID_ARG, "probs is NULL");
        TAV_NEED(c, ((uintptr_t)probs & 15) == 0, TAV_ERR_INVALID_ARG,
                 "probs is not 16-byte aligned");
        TAV_NEED(c, draft_tokens, TAV_ERR_INVALID_ARG, "draft_tokens is NULL");
        TAV_NEED(c, parents, TAV_ERR_INVALID_ARG, "parents is NULL");
        TAV_NEED(c, coins, TAV_ERR_INVALID_ARG, "coins is NULL");
        TAV_NEED(c, bonus_u, TAV_ERR_INVALID_ARG, "bonus_u is NULL");
        TAV_NEED(c, accepted_path, TAV_ERR_INVALID_ARG, "accepted_path is NULL");
        TAV_NEED(c, accept_len, TAV_ERR_INVALID_ARG, "accept_len is NULL");
        if (c.status == TAV_OK) {
            const RejPlan p = rej_plan(B, V);
            TAV_NEED(c, workspace, TAV_ERR_WORKSPACE, "workspace is NULL");
            TAV_NEED(c, ((uintptr_t)workspace & 255) == 0, TAV_ERR_WORKSPACE,
                     "workspace is not 256-byte aligned");
            TAV_NEED(c, workspace_bytes >= p.bytes, TAV_ERR_WORKSPACE,
                     "workspace too small: " + str((long long)workspace_bytes) + " < " +
                         str((long long)p.bytes) + " bytes");
        }
    }
    if (c.status != TAV_OK || B == 0)
        return tav::finish("verify_tree_rejection", c);
    const RejPlan p = rej_plan(B, V);
    char *ws = (char *)workspace;
    // the ticket counter and every request's job counters start at zero
    const int64_t n16 = (int64_t)(p.zero_bytes / 16);
    const int cblocks = (int)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
    hipLaunchKernelGGL(k_rej_clear, dim3((unsigned)cblocks), dim3(256), 0, S(stream), (uint4 *)ws,
                       n16);
    tav_status st = tav::launched("verify_tree_rejection");
    if (st != TAV_OK)
        return st;
    RejArgs a{};
    a.probs = probs;
    a.row_stride = row_stride;
    a.q = draft_q;
    a.q_row_stride = q_row_stride;
    a.V = V;
    a.N = N;
    a.B = B;
    a.nslices = p.nslices;
    a.draft = draft_tokens;
    a.parents = parents;
    a.score = draft_score;
    a.coins = coins;
    a.bonus_u = bonus_u;
    a.path = accepted_path;
    a.accept_len = accept_len;
    a.tokens = accepted_tokens;
    a.G = p.G;
    a.ticket = (int *)ws;
    a.ctl = (RejCtl *)(ws + p.ctl_off);
    a.tsum = (float *)(ws + p.tsum_off);
    const dim3 grid((unsigned)(B * p.G));
    if (draft_q)
        hipLaunchKernelGGL(k_verify_rejection<true>, grid, dim3(kRejThreads), 0, S(stream), a);
    else
        hipLaunchKernelGGL(k_verify_rejection<false>, grid, dim3(kRejThreads), 0, S(stream), a);
    return tav::launched("verify_tree_rejection");
}
