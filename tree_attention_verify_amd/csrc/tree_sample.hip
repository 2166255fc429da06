// Sampled verify: Gumbel-max target draws of every verify row, keyed by
// (request seed, the position the node predicts).
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
