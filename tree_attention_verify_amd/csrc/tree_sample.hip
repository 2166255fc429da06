// Sampled verify, two ways:
//   - Gumbel-max target draws of every verify row, keyed by (request seed,
//     the position the node predicts), walked by verify_tree_greedy;
//   - tree rejection sampling of the draft tokens against the target rows
//     (k_verify_rejection, and k_verify_rejection_q against the draft
//     distribution that drew each node's children), further below.
//
// "Draft-tree speculation", section "Sampled verify keys noise by position":
// a verify row draws its target token by Gumbel-max keyed by (seed,
// position), where for a tree the position is the one the node predicts,
// vc + depth + 1, never the row; acceptance is then the greedy tree walk
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
// recursive rejection sampling is exact in distribution).  The draft tokens
// are fixed candidates: child c of node cur (token x) is accepted when
// coin[c] * (S - E) < w(x), with w the node's target row (positive finite
// entries, else 0), S its total and E the mass of the tokens already
// rejected there, which leave the residual; the walk ends with a bonus token
// drawn from the residual by inverse CDF.
//
// One workgroup of 16 waves per request.  A visited row is read once: each
// wave sums 256-token tiles (eight 1 KB tiles in flight per wave, their
// butterflies side by side), keeping every tile sum in LDS.  Meanwhile lane
// j of wave 0 loads the weight of child j's token; with the row total, wave
// 0 then tests every child at once: its rank in the trying order, whether
// its token repeats an earlier sibling's, and the weight E of the distinct
// tokens before it come from a pass over the children (readlane), and the
// accepted child is the lowest-ranked one whose test passes.  At the last
// node the tiles holding rejected tokens are summed again without them;
// wave 0 scans the tile sums to the tile where the running sum passes
// u * total, then that tile's lanes (four tokens each) to the token.
constexpr int kRejWaves = 16;
constexpr int kRejThreads = 64 * kRejWaves;
constexpr int kRejTile = 256;                    // tokens per tile: 64 lanes x 4
constexpr int kRejMaxV = 1 << 20;
constexpr int kRejMaxTiles = kRejMaxV / kRejTile;
constexpr int kRejBatch = 8;                     // tiles per wave in flight

struct RejArgs {
    const float *probs;
    int64_t row_stride;
    int32_t V, N;
    const int32_t *draft, *parents;
    const float *score, *coins, *bonus_u;
    int32_t *path, *accept_len, *tokens;
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

__global__ void __launch_bounds__(kRejThreads) k_verify_rejection(RejArgs a) {
    __shared__ float tsum[kRejMaxTiles];
    __shared__ float wpart[kRejWaves];
    __shared__ int32_t s_par[64], s_dr[64], s_path[64], s_rej[64];
    __shared__ float s_sc[64], s_coin[64], s_bu[64];
    __shared__ int s_next, s_nrej, s_bonus;

    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = a.N, V = a.V;
    const int64_t nb = (int64_t)b * N;
    if (tid < N) {
        s_par[tid] = a.parents[nb + tid];
        s_dr[tid] = a.draft[nb + tid];
        s_sc[tid] = a.score ? a.score[nb + tid] : 0.f;
        s_coin[tid] = a.coins[nb + tid];
        s_bu[tid] = a.bonus_u[nb + tid];
    }
    if (tid == 0)
        s_path[0] = 0;
    __syncthreads();

    const int ntiles = (V + kRejTile - 1) / kRejTile;
    const int nfull = V / kRejTile;   // whole tiles
    int cur = 0, len = 1;
    const float *row;
    for (;;) {
        row = a.probs + (nb + cur) * a.row_stride;
        // wave 0, lane j = node j: a child's token weight, loaded before the
        // row's pass so that its latency overlaps it
        const bool is_child = w == 0 && lane < N && len < N && s_par[lane] == cur;
        const int xj = lane < N ? s_dr[lane] : -1;
        const bool valid = is_child && xj >= 0 && xj < V;
        const float wx = valid ? rej_w(row[xj]) : 0.f;
        // tile sums of the row and this wave's share of the total: whole
        // tiles with unconditional loads (a batch past the end rereads the
        // last whole tile and drops it), then the partial tile
        float acc = 0.f;
        for (int t0 = w * kRejBatch; t0 < nfull; t0 += kRejWaves * kRejBatch) {
            float4 x[kRejBatch];
#pragma unroll
            for (int i = 0; i < kRejBatch; ++i)
                x[i] = *(const float4 *)(row + min(t0 + i, nfull - 1) * kRejTile + lane * 4);
            // the batch's butterflies side by side (the same sums as
            // rej_wave_sum, one wait per step instead of one per tile)
            float ls[kRejBatch];
#pragma unroll
            for (int i = 0; i < kRejBatch; ++i)
                ls[i] = (rej_w(x[i].x) + rej_w(x[i].y)) + (rej_w(x[i].z) + rej_w(x[i].w));
#pragma unroll
            for (int m = 1; m < 64; m <<= 1)
#pragma unroll
                for (int i = 0; i < kRejBatch; ++i)
                    ls[i] += __shfl_xor(ls[i], m, 64);
#pragma unroll
            for (int i = 0; i < kRejBatch; ++i) {
                if (t0 + i < nfull) {
                    if (lane == 0)
                        tsum[t0 + i] = ls[i];
                    acc += ls[i];
                }
            }
        }
        if (nfull < ntiles && w == kRejWaves - 1) {
            const int v0 = nfull * kRejTile + lane * 4;
            float r[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                r[e] = v0 + e < V ? rej_w(row[v0 + e]) : 0.f;
            const float s = rej_wave_sum((r[0] + r[1]) + (r[2] + r[3]));
            if (lane == 0)
                tsum[nfull] = s;
            acc += s;
        }
        if (lane == 0)
            wpart[w] = acc;
        __syncthreads();
        if (w == 0) {
            float S = 0.f;
            for (int i = 0; i < kRejWaves; ++i)
                S += wpart[i];
            // Siblings are tried in descending draft score, the lower index on
            // ties: child j's rank counts the children before it, E_j the
            // weight of the distinct valid tokens before it (all rejected if
            // the walk reaches j), and a token repeating an earlier sibling's
            // has no residual weight.
            const float scj = lane < N ? s_sc[lane] : 0.f;
            const uint64_t cm = __ballot(is_child), vmask = __ballot(valid);
            auto lane_f = [](float v, int i) {
                return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), i));
            };
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
            const bool pass = is_child && s_coin[lane < N ? lane : 0] * (S - Ej) < wxe;
            // the first passing child in the trying order
            int best = pass ? rank : 64;
#pragma unroll
            for (int m = 1; m < 64; m <<= 1)
                best = min(best, __shfl_xor(best, m, 64));
            const uint64_t win = __ballot(pass && rank == best);
            const int next = win ? __builtin_ctzll(win) : -1;
            // tokens rejected at this node when the walk stops here: every
            // valid child token
            const uint64_t vm = __ballot(valid);
            if (valid)
                s_rej[__builtin_popcountll(vm & ((1ull << lane) - 1))] = xj;
            if (lane == 0) {
                s_next = next;
                s_nrej = next >= 0 ? 0 : __builtin_popcountll(vm);
                if (next >= 0)
                    s_path[len] = next;
            }
        }
        __syncthreads();
        const int next = s_next;
        if (next < 0)
            break;
        cur = next;
        ++len;
    }

    // the bonus: tiles holding rejected tokens summed again without them
    const int nrej = s_nrej;
    for (int i = w; i < nrej; i += kRejWaves) {
        const int t = s_rej[i] / kRejTile;
        const int v0 = t * kRejTile + lane * 4;
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int v = v0 + e;
            r[e] = v < V ? rej_w(row[v]) : 0.f;
            for (int k = 0; k < nrej; ++k)
                r[e] = s_rej[k] == v ? 0.f : r[e];
        }
        const float s = rej_wave_sum((r[0] + r[1]) + (r[2] + r[3]));
        if (lane == 0)
            tsum[t] = s;   // waves sharing a tile write the same value
    }
    __syncthreads();
    if (w == 0) {
        // running sums over the tiles, 64 at a time, the same arithmetic in
        // both passes
        float run = 0.f;
        for (int t0 = 0; t0 < ntiles; t0 += 64) {
            const float x = t0 + lane < ntiles ? tsum[t0 + lane] : 0.f;
            run += __shfl(rej_wave_scan(x, lane), 63, 64);
        }
        const float total = run;
        const float target = s_bu[cur] * total;
        int k = -1, last = -1;
        float before = 0.f;
        run = 0.f;
        for (int t0 = 0; t0 < ntiles && k < 0; t0 += 64) {
            const float x = t0 + lane < ntiles ? tsum[t0 + lane] : 0.f;
            const float inc = rej_wave_scan(x, lane);
            const float up = __shfl_up(inc, 1, 64);
            const float exc = lane > 0 ? up : 0.f;
            const uint64_t pass = __ballot(run + inc > target && x > 0.f);
            const uint64_t pos = __ballot(x > 0.f);
            if (pos)
                last = t0 + 63 - __builtin_clzll(pos);
            if (pass) {
                const int l = __builtin_ctzll(pass);
                k = t0 + l;
                before = run + __shfl(exc, l, 64);
            }
            run += __shfl(inc, 63, 64);
        }
        int bonus = 0;
        if (total > 0.f) {
            const bool crossed = k >= 0;
            if (!crossed)
                k = last;
            // tile k: lane l holds its tokens 4 l .. 4 l + 3 (rejected ones
            // zeroed); the first lane whose running sum passes the target
            // scans its four
            const int v0 = k * kRejTile + lane * 4;
            float r[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int v = v0 + e;
                r[e] = v < V ? rej_w(row[v]) : 0.f;
                for (int j = 0; j < nrej; ++j)
                    r[e] = s_rej[j] == v ? 0.f : r[e];
            }
            const float ls = ((r[0] + r[1]) + r[2]) + r[3];
            const float inc = rej_wave_scan(ls, lane);
            const float up = __shfl_up(inc, 1, 64);
            const float exc = lane > 0 ? up : 0.f;
            const uint64_t hit = __ballot(crossed && ls > 0.f && before + inc > target);
            const uint64_t nz = __ballot(ls > 0.f);
            // no lane passes only through rounding: the tile's last positive token
            const int l = hit ? __builtin_ctzll(hit) : (nz ? 63 - __builtin_clzll(nz) : 0);
            int e_pick = -1, e_last = -1;
            float cum = before + exc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (r[e] > 0.f) {
                    e_last = e;
                    cum += r[e];
                    if (hit && e_pick < 0 && cum > target)
                        e_pick = e;
                }
            }
            const int e_sel = e_pick >= 0 ? e_pick : e_last;
            bonus = k * kRejTile + 4 * l + __shfl(e_sel < 0 ? 0 : e_sel, l, 64);
        }
        if (lane == 0)
            s_bonus = bonus;
    }
    __syncthreads();
    if (tid < N) {
        const int p = tid < len ? s_path[tid] : -1;
        a.path[nb + tid] = p;
        if (a.tokens)
            a.tokens[nb + tid] = tid + 1 < len ? s_dr[s_path[tid + 1]] : (tid + 1 == len ? s_bonus : -1);
    }
    if (tid == 0)
        a.accept_len[b] = len;
}

// The walk against the draft distribution q that drew each node's children
// ("Draft-tree speculation", section "Sampled verify keys noise by
// position": recursive rejection sampling against that q, exact in
// distribution).  At node cur the residual starts as r_0 = w / S and q^ =
// q / Q (positive finite entries); child i (token x) in the trying order is
// accepted when coin * q^(x) < r_i(x), else r_{i+1} = max(0, r_i - q^) /
// Z_{i+1}.  r_i(v) depends only on w(v), q(v), S, Q and Z_1 .. Z_i, so a
// test reads two floats and each rejection costs one pass over both rows
// for the next Z; the bonus draws from the final residual through tile sums
// as in k_verify_rejection.
struct RejQArgs {
    RejArgs a;
    const float *q;
    int64_t q_row_stride;
};

__global__ void __launch_bounds__(kRejThreads) k_verify_rejection_q(RejQArgs qa) {
    const RejArgs &a = qa.a;
    __shared__ float tsum[kRejMaxTiles];
    __shared__ float red[2][kRejWaves];
    __shared__ float zinv[64];                    // 1 / Z_1 .. 1 / Z_k at the current node (0: none left)
    __shared__ int32_t s_par[64], s_dr[64], s_path[64], s_ord[64];
    __shared__ float s_sc[64], s_coin[64], s_bu[64];
    __shared__ int s_nk, s_acc, s_bonus;

    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = a.N, V = a.V;
    const int64_t nb = (int64_t)b * N;
    if (tid < N) {
        s_par[tid] = a.parents[nb + tid];
        s_dr[tid] = a.draft[nb + tid];
        s_sc[tid] = a.score ? a.score[nb + tid] : 0.f;
        s_coin[tid] = a.coins[nb + tid];
        s_bu[tid] = a.bonus_u[nb + tid];
    }
    if (tid == 0)
        s_path[0] = 0;
    __syncthreads();

    // the sum over the workgroup, the same value in every thread
    auto block_sum2 = [&](float x, float y, float &sx, float &sy) {
        x = rej_wave_sum(x);
        y = rej_wave_sum(y);
        if (lane == 0) {
            red[0][w] = x;
            red[1][w] = y;
        }
        __syncthreads();
        sx = 0.f;
        sy = 0.f;
        for (int i = 0; i < kRejWaves; ++i) {
            sx += red[0][i];
            sy += red[1][i];
        }
        __syncthreads();
    };

    const int ntiles = (V + kRejTile - 1) / kRejTile;
    int cur = 0, len = 1, nrej = 0;
    float S = 0.f, Q = 0.f, iS = 0.f, iQ = 0.f;
    const float *row, *qrow;
    // the residual after k rejections at token v
    // f(p[v], q[v]) for every token of the two rows of node cur: 16-byte
    // loads, four of each row in flight per thread, then the tail
    auto over_rows = [&](auto f) {
        const int V4 = V >> 2;
        constexpr int U = 4;
        for (int i0 = tid; i0 < V4; i0 += U * kRejThreads) {
            float4 pv[U], qv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = min(i0 + u * kRejThreads, V4 - 1);
                pv[u] = reinterpret_cast<const float4 *>(row)[i];
                qv[u] = reinterpret_cast<const float4 *>(qrow)[i];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (i0 + u * kRejThreads < V4) {
                    f(pv[u].x, qv[u].x);
                    f(pv[u].y, qv[u].y);
                    f(pv[u].z, qv[u].z);
                    f(pv[u].w, qv[u].w);
                }
            }
        }
        for (int v = 4 * V4 + tid; v < V; v += kRejThreads)
            f(row[v], qrow[v]);
    };
    // (reciprocals of the totals and normalisers, computed once each)
    auto resid = [&](float pv, float qv, int k) {
        float r = rej_w(pv) * iS;
        const float qh = rej_w(qv) * iQ;
        for (int j = 0; j < k; ++j)
            r = fmaxf(r - qh, 0.f) * zinv[j];
        return r;
    };
    for (;;) {
        row = a.probs + (nb + cur) * a.row_stride;
        qrow = qa.q + (nb + cur) * qa.q_row_stride;
        float sp = 0.f, sq = 0.f;
        over_rows([&](float pv, float qv) {
            sp += rej_w(pv);
            sq += rej_w(qv);
        });
        block_sum2(sp, sq, S, Q);
        iS = S > 0.f ? 1.f / S : 0.f;
        iQ = Q > 0.f ? 1.f / Q : 0.f;
        // the children in their trying order (wave 0, as k_verify_rejection)
        if (w == 0) {
            const bool is_child = lane < N && len < N && s_par[lane] == cur;
            const float scj = lane < N ? s_sc[lane] : 0.f;
            const uint64_t cm = __ballot(is_child);
            int rank = 0;
            for (uint64_t m = cm; m; m &= m - 1) {
                const int i = __builtin_ctzll(m);
                const float sci = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(scj), i));
                rank += (sci > scj || (sci == scj && i < lane)) ? 1 : 0;
            }
            if (is_child)
                s_ord[rank] = lane;
            if (lane == 0)
                s_nk = __builtin_popcountll(cm);
        }
        __syncthreads();
        const int nk = s_nk;
        int next = -1;
        nrej = 0;
        for (int i = 0; i < nk; ++i) {
            const int c = s_ord[i];
            if (tid == 0) {
                const int x = s_dr[c];
                bool acc = false;
                if (x >= 0 && x < V) {
                    acc = s_coin[c] * (rej_w(qrow[x]) * iQ) < resid(row[x], qrow[x], i);
                }
                s_acc = acc;
            }
            __syncthreads();
            if (s_acc) {
                next = c;
                break;
            }
            // rejected: Z_{i+1} = sum_v max(0, r_i(v) - q^(v))
            float z = 0.f;
            over_rows([&](float pv, float qv) { z += fmaxf(resid(pv, qv, i) - rej_w(qv) * iQ, 0.f); });
            float z_all, unused;
            block_sum2(z, 0.f, z_all, unused);
            if (tid == 0)
                zinv[i] = z_all > 0.f ? 1.f / z_all : 0.f;
            nrej = i + 1;
            __syncthreads();
        }
        if (next < 0)
            break;
        if (tid == 0)
            s_path[len] = next;
        cur = next;
        ++len;
        __syncthreads();
    }

    // the bonus from r_nrej: tile sums (whole tiles by unconditional 16-byte
    // loads, four tiles in flight per wave, then the partial tile), then the
    // tile, then the token
    const int nfull = V / kRejTile;
    for (int t0 = w * 4; t0 < nfull; t0 += kRejWaves * 4) {
        float4 pv[4], qv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int off = min(t0 + i, nfull - 1) * kRejTile + lane * 4;
            pv[i] = *(const float4 *)(row + off);
            qv[i] = *(const float4 *)(qrow + off);
        }
        float ls[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ls[i] = (resid(pv[i].x, qv[i].x, nrej) + resid(pv[i].y, qv[i].y, nrej)) +
                    (resid(pv[i].z, qv[i].z, nrej) + resid(pv[i].w, qv[i].w, nrej));
#pragma unroll
        for (int m = 1; m < 64; m <<= 1)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ls[i] += __shfl_xor(ls[i], m, 64);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (t0 + i < nfull && lane == 0)
                tsum[t0 + i] = ls[i];
    }
    if (nfull < ntiles && w == kRejWaves - 1) {
        const int v0 = nfull * kRejTile + lane * 4;
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            r[e] = v0 + e < V ? resid(row[v0 + e], qrow[v0 + e], nrej) : 0.f;
        const float s = rej_wave_sum((r[0] + r[1]) + (r[2] + r[3]));
        if (lane == 0)
            tsum[nfull] = s;
    }
    __syncthreads();
    if (w == 0) {
        float run = 0.f;
        for (int t0 = 0; t0 < ntiles; t0 += 64) {
            const float x = t0 + lane < ntiles ? tsum[t0 + lane] : 0.f;
            run += __shfl(rej_wave_scan(x, lane), 63, 64);
        }
        const float total = run;
        const float target = s_bu[cur] * total;
        int k = -1, last = -1;
        float before = 0.f;
        run = 0.f;
        for (int t0 = 0; t0 < ntiles && k < 0; t0 += 64) {
            const float x = t0 + lane < ntiles ? tsum[t0 + lane] : 0.f;
            const float inc = rej_wave_scan(x, lane);
            const float up = __shfl_up(inc, 1, 64);
            const float exc = lane > 0 ? up : 0.f;
            const uint64_t pass = __ballot(run + inc > target && x > 0.f);
            const uint64_t pos = __ballot(x > 0.f);
            if (pos)
                last = t0 + 63 - __builtin_clzll(pos);
            if (pass) {
                const int l = __builtin_ctzll(pass);
                k = t0 + l;
                before = run + __shfl(exc, l, 64);
            }
            run += __shfl(inc, 63, 64);
        }
        int bonus = 0;
        if (total > 0.f) {
            const bool crossed = k >= 0;
            if (!crossed)
                k = last;
            const int v0 = k * kRejTile + lane * 4;
            float r[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                r[e] = v0 + e < V ? resid(row[v0 + e], qrow[v0 + e], nrej) : 0.f;
            const float ls = ((r[0] + r[1]) + r[2]) + r[3];
            const float inc = rej_wave_scan(ls, lane);
            const float up = __shfl_up(inc, 1, 64);
            const float exc = lane > 0 ? up : 0.f;
            const uint64_t hit = __ballot(crossed && ls > 0.f && before + inc > target);
            const uint64_t nz = __ballot(ls > 0.f);
            const int l = hit ? __builtin_ctzll(hit) : (nz ? 63 - __builtin_clzll(nz) : 0);
            int e_pick = -1, e_last = -1;
            float cum = before + exc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (r[e] > 0.f) {
                    e_last = e;
                    cum += r[e];
                    if (hit && e_pick < 0 && cum > target)
                        e_pick = e;
                }
            }
            const int e_sel = e_pick >= 0 ? e_pick : e_last;
            bonus = k * kRejTile + 4 * l + __shfl(e_sel < 0 ? 0 : e_sel, l, 64);
        }
        if (lane == 0)
            s_bonus = bonus;
    }
    __syncthreads();
    if (tid < N) {
        a.path[nb + tid] = tid < len ? s_path[tid] : -1;
        if (a.tokens)
            a.tokens[nb + tid] = tid + 1 < len ? s_dr[s_path[tid + 1]] : (tid + 1 == len ? s_bonus : -1);
    }
    if (tid == 0)
        a.accept_len[b] = len;
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
    c.need(B >= 0, TAV_ERR_INVALID_ARG, "B must be >= 0, got " + str(B));
    c.need(N >= 1 && N <= 64, TAV_ERR_INVALID_ARG, "N must be in [1, 64], got " + str(N));
    c.need(V >= 1, TAV_ERR_INVALID_ARG, "V must be >= 1, got " + str(V));
    c.need(dtype == TAV_BF16 || dtype == TAV_F32, TAV_ERR_UNSUPPORTED,
           "logits dtype must be TAV_BF16 or TAV_F32, got " + str(dtype));
    const int elem = dtype == TAV_F32 ? 4 : 2;
    c.need(row_stride >= V, TAV_ERR_INVALID_ARG,
           "row_stride must be >= V, got " + str(row_stride) + " < " + str(V));
    c.need((row_stride * elem) % 16 == 0, TAV_ERR_INVALID_ARG,
           "row_stride must span a multiple of 16 bytes, got " + str(row_stride) + " elements");
    c.need((long long)B * N * row_stride < (1LL << 62), TAV_ERR_INVALID_ARG, "logits too large");
    if (B > 0) {
        c.need(logits, TAV_ERR_INVALID_ARG, "logits is NULL");
        c.need(((uintptr_t)logits & 15) == 0, TAV_ERR_INVALID_ARG, "logits is not 16-byte aligned");
        c.need(temperature, TAV_ERR_INVALID_ARG, "temperature is NULL");
        c.need(seed, TAV_ERR_INVALID_ARG, "seed is NULL");
        c.need(positions, TAV_ERR_INVALID_ARG, "positions is NULL");
        c.need(tokens, TAV_ERR_INVALID_ARG, "tokens is NULL");
        if (c.status == TAV_OK) {
            const SamplePlan p = sample_plan(B, N, V);
            c.need(workspace, TAV_ERR_WORKSPACE, "workspace is NULL");
            c.need(((uintptr_t)workspace & 255) == 0, TAV_ERR_WORKSPACE,
                   "workspace is not 256-byte aligned");
            c.need(workspace_bytes >= p.bytes, TAV_ERR_WORKSPACE,
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

extern "C" tav_status verify_tree_rejection(const float *probs, int64_t row_stride, int32_t V,
                                            const float *draft_q, int64_t q_row_stride,
                                            const int32_t *draft_tokens, const int32_t *parents,
                                            const float *draft_score, const float *coins,
                                            const float *bonus_u, int32_t B, int32_t N,
                                            int32_t *accepted_path, int32_t *accept_len,
                                            int32_t *accepted_tokens, void *stream) {
    Checks c;
    c.need(B >= 0, TAV_ERR_INVALID_ARG, "B must be >= 0, got " + str(B));
    c.need(N >= 1 && N <= 64, TAV_ERR_INVALID_ARG, "N must be in [1, 64], got " + str(N));
    c.need(V >= 1 && V <= kRejMaxV, TAV_ERR_INVALID_ARG,
           "V must be in [1, " + str(kRejMaxV) + "], got " + str(V));
    c.need(row_stride >= V, TAV_ERR_INVALID_ARG,
           "row_stride must be >= V, got " + str(row_stride) + " < " + str(V));
    c.need(row_stride % 4 == 0, TAV_ERR_INVALID_ARG,
           "row_stride must be a multiple of 4 elements, got " + str(row_stride));
    c.need((long long)B * N * row_stride < (1LL << 62), TAV_ERR_INVALID_ARG, "probs too large");
    if (draft_q) {
        c.need(q_row_stride >= V, TAV_ERR_INVALID_ARG,
               "q_row_stride must be >= V, got " + str(q_row_stride) + " < " + str(V));
        c.need(q_row_stride % 4 == 0, TAV_ERR_INVALID_ARG,
               "q_row_stride must be a multiple of 4 elements, got " + str(q_row_stride));
        c.need(((uintptr_t)draft_q & 15) == 0, TAV_ERR_INVALID_ARG, "draft_q is not 16-byte aligned");
        c.need((long long)B * N * q_row_stride < (1LL << 62), TAV_ERR_INVALID_ARG, "draft_q too large");
    }
    if (B > 0) {
        c.need(probs, TAV_ERR_INVALID_ARG, "probs is NULL");
        c.need(((uintptr_t)probs & 15) == 0, TAV_ERR_INVALID_ARG, "probs is not 16-byte aligned");
        c.need(draft_tokens, TAV_ERR_INVALID_ARG, "draft_tokens is NULL");
        c.need(parents, TAV_ERR_INVALID_ARG, "parents is NULL");
        c.need(coins, TAV_ERR_INVALID_ARG, "coins is NULL");
        c.need(bonus_u, TAV_ERR_INVALID_ARG, "bonus_u is NULL");
        c.need(accepted_path, TAV_ERR_INVALID_ARG, "accepted_path is NULL");
        c.need(accept_len, TAV_ERR_INVALID_ARG, "accept_len is NULL");
    }
    if (c.status != TAV_OK || B == 0)
        return tav::finish("verify_tree_rejection", c);
    RejArgs a{};
    a.probs = probs;
    a.row_stride = row_stride;
    a.V = V;
    a.N = N;
    a.draft = draft_tokens;
    a.parents = parents;
    a.score = draft_score;
    a.coins = coins;
    a.bonus_u = bonus_u;
    a.path = accepted_path;
    a.accept_len = accept_len;
    a.tokens = accepted_tokens;
    if (draft_q) {
        RejQArgs qa{a, draft_q, q_row_stride};
        hipLaunchKernelGGL(k_verify_rejection_q, dim3((unsigned)B), dim3(kRejThreads), 0, S(stream),
                           qa);
    } else {
        hipLaunchKernelGGL(k_verify_rejection, dim3((unsigned)B), dim3(kRejThreads), 0, S(stream),
                           a);
    }
    return tav::launched("verify_tree_rejection");
}
