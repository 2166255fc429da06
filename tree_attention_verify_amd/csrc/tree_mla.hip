// tree_attention_mla: the verify cascade over an MLA latent cache, for gfx950.
//
// "Draft-tree speculation", section "One tree attention ...", the MLA
// paragraph: the cascade is unchanged, only the key and value differ.  Each
// token keeps one latent row shared by all query heads: its first Dc
// channels score against the query's first Dc channels and are also the
// value, and its Dr rotary channels add a second dot product to the score.
// All R x Hq query rows of a request are therefore folded into the MFMA N
// dimension against one stream of latent rows, each read once.  Under an
// FP8 E4M3 latent cache the query is rounded to E4M3 for every key (the
// page's window kernel receives the FP8 query) and the rows are widened to
// bf16 exactly.
//
// Kernels:
//   k_mla_prefix<DR>  split-K prefix decode.  One workgroup of 8 waves (two
//       per SIMD, at most 256 registers each) owns 64 folded rows and all
//       Dc = 512 value channels.  Per 32-key block each wave first scores one
//       16-row x 16-key tile over the Dc + Dr channels (18 steps of
//       v_mfma_f32_16x16x32_bf16 for Dr = 64, the query of its 16 rows in
//       registers) and writes its bf16 weights to LDS; after a barrier each
//       wave accumulates O^T += V^T P^T for 64 value channels of all 64 rows
//       (16 MFMAs).  Every score is computed once.  Latent rows stream HBM ->
//       LDS with direct-to-LDS 16-byte loads, four stages deep; the same LDS
//       bytes are read as the K operand and, transposed, as the V operand.
//       FP8 rows land raw in a ring of two slots (in the space of the fourth
//       stage buffer); at the end of a trip each lane takes the chunks it
//       loaded into registers, and at the top of the next it widens them
//       into the bf16 layout of a stage buffer (the bf16 stages ring over
//       three) and issues the slot's next raw stage.
//   k_mla_window_merge<DR>  one wave per (request, row, head): the masked
//       window keys (never the unseen ones) with lanes over channels, then
//       the merge of the prefix partials through their base-2 LSE.
//
// LDS layout of a stage of 32 keys: 1 KB blocks [chunk group G][key block
// K8] (G = 8 consecutive 16-byte chunks of the row, K8 = 8 consecutive
// keys); inside a block key k owns the 128-byte row 128 (k % 8), its chunk c
// at 16-byte slot (c % 8) ^ (k % 8).  Measured on gfx950: the K operand read
// (16 keys x 4 chunks) and the transposing V read (16 keys x 2 chunks) both
// run at the full LDS rate with this swizzle, and the direct-to-LDS loads,
// eight lanes per 128-byte row segment, at the full L2 -> LDS rate; a layout
// with consecutive lanes on different rows (which kept the LDS reads as fast)
// loaded at about a quarter of it.
#include <cmath>

#include "tav_internal.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
#define MLA_LDS __attribute__((address_space(3)))

constexpr float kLog2eM = 1.4426950408889634f;
constexpr int kMlaPt = 1024;            // page-table entries one split may span

__device__ inline uint16_t mla_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Direct-to-LDS 16-byte load: lane i's 16 bytes land at LDS byte lds_base +
// 16 i; completion by vmcnt then a workgroup barrier (see the prefix kernel
// of tree_attention.hip for why it is inline assembly).
__device__ __forceinline__ void mla_dma16(const void *src, uint32_t lds_base) {
    int m0v;   // m0 is an output, so the compiler keeps no value of its own there
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
                 : "={m0}"(m0v)
                 : "v"(src), "s"(lds_base)
                 : "memory");
}

template <int N>
__device__ inline void mla_wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <typename T>
__device__ __forceinline__ void mla_settle(T &x) {
    asm volatile("" : "+v"(x));
}

// max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one row of a
// 16 x 16 MFMA result)
__device__ inline float mla_quad_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ inline float mla_quad_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// FP8 E4M3 latent caches.  Every E4M3 value (NaN included) is a bf16 value,
// so widening is exact: a 16-byte chunk of 16 codes becomes two bf16 chunks.
__device__ __forceinline__ void mla_fp8x16_to_bf16(const int4 x, int4 &lo, int4 &hi) {
    auto c0 = [](int w) {
        return __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w, 1.0f, false));
    };
    auto c1 = [](int w) {
        return __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w, 1.0f, true));
    };
    lo = make_int4(c0(x.x), c1(x.x), c0(x.y), c1(x.y));
    hi = make_int4(c0(x.z), c1(x.z), c0(x.w), c1(x.w));
}

// x rounded to the nearest E4M3 value (ties to even) as fp32; magnitudes past
// 448 give +-448, NaN stays NaN.  Above the subnormal range an E4M3 value has
// 4 significant bits (quantum 2^(e - 3) at binary exponent e), below 2^-6 the
// quantum is 2^-9; the scalings are exact and rint rounds ties to even.
__device__ inline float mla_round_e4m3(float x) {
    if (!(fabsf(x) <= 448.f))
        return x != x ? x : copysignf(448.f, x);
    const float a = fabsf(x);
    int e = (int)((__float_as_uint(a) >> 23) & 0xff) - 127;
    e = e < -6 ? -6 : e;
    const float up = __uint_as_float((uint32_t)(3 - e + 127) << 23);
    const float dn = __uint_as_float((uint32_t)(e - 3 + 127) << 23);
    return copysignf(__builtin_rintf(a * up) * dn, x);
}

// eight bf16 values (raw bits in an int4) rounded to E4M3, held as bf16
// (exact: every E4M3 value is a bf16 value)
__device__ inline int4 mla_bf16x8_round_e4m3(int4 v) {
    uint32_t u[4] = {(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float lo = mla_round_e4m3(__uint_as_float(u[e] << 16));
        const float hi = mla_round_e4m3(__uint_as_float(u[e] & 0xffff0000u));
        u[e] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
    }
    return make_int4((int)u[0], (int)u[1], (int)u[2], (int)u[3]);
}

struct MlaArgs {
    const uint16_t *q;
    const uint16_t *lat;
    int64_t stride_page, stride_token, num_pages;
    const int32_t *page_table;
    int32_t max_pages, ps_shift;
    const int32_t *prefix_len;
    int32_t max_prefix_len;
    const uint64_t *masks;
    int32_t W, B, R, Hq, M, RG, n_split, kps;
    float c;        // sm_scale * log2(e)
    float *ws_o;    // [rows][n_split][512]
    float *ws_lse;  // [rows][n_split]
    uint16_t *out;  // [B][R][Hq][512]
    float *lse2;    // [B][R][Hq] or null
};

template <int DR>
struct MlaCfg {
    static constexpr int DC = 512;
    static constexpr int DK = DC + DR;
    static constexpr int KS = DK / 32;             // 32-channel score steps
    static constexpr int NG = DK / 64;             // 8-chunk groups per row
    static constexpr int SK = 32;                  // keys per stage
    static constexpr int SB = NG * SK * 128;       // stage bytes
    static constexpr int NBUF = 4;
    static constexpr int LOADS = NG * SK * 8 / 64; // load instructions per stage (64 lanes each)
    static constexpr int LA = (NG + 1) / 2;        // loads per stage of waves 0..3
    static constexpr int LB = NG - LA;             // and of waves 4..7
    static constexpr int PB = 64 * SK * 2;         // bf16 weights of a block: 64 rows x 32 keys
    // FP8 E4M3 rows (DK bytes): raw stages of SK rows land in a ring of two
    // slots in the space of the fourth stage buffer (the bf16 stages then
    // ring over three): 32 chunks of 16 bytes a row in two load instructions
    // per wave (keys 4 w .. 4 w + 3), the rotary part's 4 chunks a row in one
    // more for waves 0 and 1 (16 keys each)
    static constexpr int CH8 = DK / 16;            // 16-byte chunks per FP8 row
    static constexpr int NB8 = 3;                  // bf16 stage buffers under FP8 rows
    static constexpr int RAW8 = NB8 * SB;          // byte offset of the raw ring
    static_assert(DK % 64 == 0 && LOADS == 4 * NG && KS >= 2 * LA, "row shape");
    static_assert(SK == 32 && (CH8 == 32 || CH8 == 36) && 2 * SK * DK <= SB, "fp8 rows");
    static_assert(NBUF * SB + 2 * PB + kMlaPt * 4 + 3 * 2 * 64 * 4 <= 160 * 1024, "LDS");
};

template <int DR, bool KV8>
__global__ void __launch_bounds__(512, 1) k_mla_prefix(MlaArgs a) {
    using C = MlaCfg<DR>;
    constexpr int DK = C::DK, KS = C::KS, SK = C::SK, SB = C::SB, NBUF = C::NBUF, LA = C::LA, LB = C::LB;
    constexpr int NB = KV8 ? C::NB8 : NBUF;   // stage buffers the bf16 stages ring over
    __shared__ __attribute__((aligned(16))) char lds[NBUF * SB];
    __shared__ __attribute__((aligned(16))) char pbuf[2 * C::PB];   // weights of blocks u, u + 1
    __shared__ int32_t pt[kMlaPt];
    __shared__ float xrow[3][2][64];   // per-row exchange between the two key tiles

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, i16 = lane & 15;
    // Score role: row tile rt (16 rows) x key tile kt (16 keys of each block).
    // Value role: channels 64 w .. 64 w + 63 for all 64 rows.
    const int rt = w & 3, kt = w >> 2;
    // A stream U = (request, split) has RG workgroups (64-row groups); they
    // take blocks 8 (RG (U / 8) + rg) + U % 8.  Blocks are dealt to the eight
    // XCDs in turn, so every reader of a stream's latent rows sits on XCD
    // U % 8 and one L2 serves them all.
    const int id = blockIdx.x;
    const int U = ((id >> 3) / a.RG) * 8 + (id & 7);
    const int rg = (id >> 3) % a.RG;
    if (U >= a.B * a.n_split)
        return;   // uniform per workgroup, before any barrier
    const int split = U % a.n_split;
    const int b = U / a.n_split;

    int P = a.prefix_len[b];
    P = P < 0 ? 0 : (P > a.max_prefix_len ? a.max_prefix_len : P);
    const int lo = split * a.kps;
    const int hi = min(P, lo + a.kps) > lo ? min(P, lo + a.kps) : lo;
    const int nkeys = hi - lo;
    const int ns = (nkeys + SK - 1) / SK;

    const int lp0 = nkeys > 0 ? (lo >> a.ps_shift) : 0;
    const int npt = nkeys > 0 ? ((hi - 1) >> a.ps_shift) - lp0 + 1 : 0;
    for (int i = tid; i < npt && i < kMlaPt; i += 512) {
        int64_t p = a.page_table[(int64_t)b * a.max_pages + lp0 + i];
        pt[i] = (int32_t)(p < 0 ? 0 : (p >= a.num_pages ? a.num_pages - 1 : p));
    }
    // keys past the split end are never loaded: their slots must hold finite
    // values (their weight is exactly 0)
    for (int i = tid; i < NBUF * SB / 16; i += 512)
        reinterpret_cast<int4 *>(lds)[i] = make_int4(0, 0, 0, 0);

    // Q^T operand of score step s: lane (g, i16) holds Q[row 16 rt + i16 of
    // the group][32 s + 8 g .. +8]; under an FP8 latent cache the query is
    // rounded to E4M3 (held as bf16), so every product with a widened E4M3
    // channel is exact
    const int m = rg * 64 + rt * 16 + i16;
    const bool row_ok = m < a.M;
    bf16x8 qv[KS];
    {
        const int r = row_ok ? m / a.Hq : 0, hh = row_ok ? m % a.Hq : 0;
        const uint16_t *qp = a.q + (((int64_t)b * a.R + r) * a.Hq + hh) * DK + 8 * g;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            int4 v4 = row_ok ? *(const int4 *)(qp + 32 * s) : make_int4(0, 0, 0, 0);
            if constexpr (KV8)
                v4 = mla_bf16x8_round_e4m3(v4);
            qv[s] = __builtin_bit_cast(bf16x8, v4);
        }
#pragma unroll
        for (int s = 0; s < KS; ++s)
            mla_settle(qv[s]);
    }
    __syncthreads();

    const uint32_t lds0 = (uint32_t)(uintptr_t)(const MLA_LDS void *)lds;
    const int ps_mask = (1 << a.ps_shift) - 1;
    // Every wave loads part of each stage.  Load x fills the 1 KB block (G =
    // x, keys 8 (w % 4) .. +7): lane i takes key 8 (w % 4) + i / 8 and chunk
    // 8 x + (i % 8 ^ i / 8), so a lane's loads of one stage all read one
    // latent row (one page lookup) and every eight lanes read one whole
    // 128-byte row segment.  Waves 0..3 take x < LA, waves 4..7 the rest.
    const int dkey = 8 * (w & 3) + (lane >> 3);
    const int dpos = (lane & 7) ^ (lane >> 3);
    const int x0 = w < 4 ? 0 : LA;
    const int nld = w < 4 ? LA : LB;
    struct Loads {
        const uint16_t *src;
        uint32_t sbase;
        bool on;
    };
    // the source row and LDS base of this lane's loads of stage st (none
    // past the split end)
    auto loads_of = [&](int st) {
        Loads r;
        const int t = lo + st * SK + dkey;
        r.on = st < ns && t < hi;
        const int64_t pg = pt[r.on ? (t >> a.ps_shift) - lp0 : 0];
        r.src = a.lat + pg * a.stride_page + (int64_t)(t & ps_mask) * a.stride_token + dpos * 8 + 64 * x0;
        r.sbase = lds0 + (uint32_t)((st % NBUF) * SB + 8 * (w & 3) * 128 + x0 * SK * 128);
        return r;
    };
    auto load_one = [&](const Loads &r, int j) {
        if (j < nld && r.on)
            mla_dma16(r.src + 64 * j, __builtin_amdgcn_readfirstlane(r.sbase + (uint32_t)(j * SK * 128)));
    };
    auto issue = [&](int st) {
        const Loads r = loads_of(st);
#pragma unroll
        for (int j = 0; j < LA; ++j)
            load_one(r, j);
    };
    // FP8 rows (DK bytes, CH8 16-byte chunks): stage st lands raw in slot st
    // % 2 of a ring of two, by direct-to-LDS loads.  Instruction 2 w + j (j =
    // 0, 1) of wave w carries chunks 16 j .. 16 j + 15 of keys 4 w .. 4 w + 3,
    // lane i taking key k8 and chunk 16 j + c8; with rotary channels (four
    // more chunks a row) instruction 16 + w of waves 0 and 1 carries chunks
    // 32 .. 35 of keys 16 w .. 16 w + 15 (lane i: key 16 w + i / 4, chunk 32 +
    // i % 4).  Lane i's 16 bytes land at byte 16 i of the instruction's 1 KB,
    // and the lane widens them itself, so one page lookup serves its main
    // loads of a stage and its chunk offsets never change.  Every eight
    // consecutive lanes take four chunks of each of two keys whose bf16 rows
    // have opposite parity (128-byte halves of the banks), so each 16-byte
    // write of widened chunks lands on eight distinct bank groups.
    constexpr int TC8 = C::CH8 - 32;
    constexpr int NT8 = TC8 ? SK * TC8 / 64 : 0;   // tail instructions a stage
    const bool tail8 = w < NT8;
    const int k8 = 4 * w + (((lane >> 2) & 1) | ((lane >> 5) << 1));
    const int c8 = (lane & 3) | (((lane >> 3) & 3) << 2);
    const int kt8 = (16 * w + (lane >> 2)) & (SK - 1);
    // byte offset in a bf16 stage of chunk cc of key k; widened chunk 2 c of
    // a row goes to slot s, chunk 2 c + 1 to slot s ^ 16 (c even or odd
    // alike), and chunks 16 further on are 4 chunk groups further
    auto bf16_slot = [](int k, int cc) {
        return (uint32_t)((cc >> 3) * (SK * 128) + (k >> 3) * 1024 + (k & 7) * 128 + (((cc & 7) ^ (k & 7)) * 16));
    };
    // A lane's fixed offsets, packed in two registers and unpacked at every
    // use from an opaque copy: computed in the loop, or hoisted out of it one
    // by one, they would hold a dozen registers through the score steps.
    const uint32_t pk8a = bf16_slot(k8, 2 * c8) | ((uint32_t)k8 << 16) | ((uint32_t)c8 << 24);
    const uint32_t pk8b = bf16_slot(kt8, 64 + 2 * (lane & 3)) | ((uint32_t)kt8 << 16);
    struct Lane8 {
        uint32_t wm, wt;   // bf16 slots of the main and tail chunks
        int k, kt, c;      // main key, tail key, main chunk
    };
    auto lane8 = [&]() {
        uint32_t x = pk8a, y = pk8b;
        mla_settle(x);
        mla_settle(y);
        return Lane8{x & 0xffffu, y & 0xffffu, (int)((x >> 16) & 0xffu), (int)(y >> 16), (int)(x >> 24)};
    };
    int4 r8[3];       // this lane's raw chunks of the next stage to widen
    int32_t pg8[2];   // pages of its keys in the next stage to load
    // the pages of stage sp's keys (main and tail) from the page table
    auto pages8 = [&](int sp) {
        if (sp >= ns)
            return;
        const Lane8 L = lane8();
        const int t = lo + sp * SK + L.k;
        pg8[0] = pt[t < hi ? (t >> a.ps_shift) - lp0 : 0];
        if (tail8) {
            const int t2 = lo + sp * SK + L.kt;
            pg8[1] = pt[t2 < hi ? (t2 >> a.ps_shift) - lp0 : 0];
        }
    };
    // stage st's raw loads into its slot (keys past the split end load nothing)
    auto issue8 = [&](int st) {
        if (st >= ns)
            return;
        const uint32_t rs = lds0 + (uint32_t)(C::RAW8 + (st & 1) * (SK * DK));
        const uint8_t *lat8 = (const uint8_t *)a.lat;
        const Lane8 L = lane8();
        const int t = lo + st * SK + L.k;
        if (t < hi) {
            const uint8_t *src = lat8 + (int64_t)pg8[0] * a.stride_page + (int64_t)(t & ps_mask) * a.stride_token + 16 * L.c;
            mla_dma16(src, __builtin_amdgcn_readfirstlane(rs + (uint32_t)(2 * w * 1024)));
            mla_dma16(src + 256, __builtin_amdgcn_readfirstlane(rs + (uint32_t)((2 * w + 1) * 1024)));
        }
        if (tail8) {
            const int t2 = lo + st * SK + L.kt;
            if (t2 < hi)
                mla_dma16(lat8 + (int64_t)pg8[1] * a.stride_page + (int64_t)(t2 & ps_mask) * a.stride_token +
                              16 * (32 + (lane & 3)),
                          __builtin_amdgcn_readfirstlane(rs + (uint32_t)((16 + w) * 1024)));
        }
    };
    // Wait for this wave's loads of stage st (the stage after it is issued;
    // when it is full, exactly its loads may stay in flight), then take this
    // lane's raw chunks of st into registers; keys past the split end (in the
    // last stage only) become zeros.
    auto take8 = [&](int st) {
        if (st + 1 < ns - 1) {
            if (tail8)
                mla_wait_vmcnt<NT8 ? 3 : 2>();
            else
                mla_wait_vmcnt<2>();
        } else {
            mla_wait_vmcnt<0>();
        }
        if (st >= ns)
            return;
        const char *raw = lds + C::RAW8 + (st & 1) * (SK * DK) + 16 * lane;
        r8[0] = *(const int4 *)(raw + 2 * w * 1024);
        r8[1] = *(const int4 *)(raw + (2 * w + 1) * 1024);
        if (tail8)
            r8[2] = *(const int4 *)(raw + (16 + w) * 1024);
        if (st == ns - 1) {
            const Lane8 L = lane8();
            if (lo + st * SK + L.k >= hi)
                r8[0] = r8[1] = make_int4(0, 0, 0, 0);
            if (tail8 && lo + st * SK + L.kt >= hi)
                r8[2] = make_int4(0, 0, 0, 0);
        }
    };
    // the taken chunks widened into the bf16 layout of stage st's buffer; the
    // barrier at the top of the next trip publishes them
    auto convert8 = [&](int st) {
        char *buf = lds + (st % NB) * SB;
        const Lane8 L = lane8();
        const uint32_t wm8 = L.wm, wt8 = L.wt;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            int4 h0, h1;
            mla_fp8x16_to_bf16(r8[j], h0, h1);
            *(int4 *)(buf + wm8 + j * (4 * SK * 128)) = h0;
            *(int4 *)(buf + (wm8 ^ 16u) + j * (4 * SK * 128)) = h1;
        }
        if (tail8) {
            int4 h0, h1;
            mla_fp8x16_to_bf16(r8[2], h0, h1);
            *(int4 *)(buf + wt8) = h0;
            *(int4 *)(buf + (wt8 ^ 16u)) = h1;
        }
    };

    // K operand of step s (score role): lane (g, i16) reads key 16 kt + i16,
    // chunk 4 s + g: block (s / 2, key / 8), row key % 8, slot (4 (s % 2) + g)
    // ^ (key % 8), which is koff's slot with bit 2 flipped for odd s; s / 2 is
    // an immediate.
    uint32_t koff;
    {
        const int key = 16 * kt + i16;
        koff = (uint32_t)((key >> 3) * 1024 + (key & 7) * 128 + ((g ^ (key & 7)) * 16));
    }
    // The weights of a block in LDS: [row tile][k group g][row i16] 16-byte
    // chunks, k slot 8 g + e holding key 4 g + e (e < 4) or 16 + 4 g + e - 4
    // (e >= 4).  A score lane (g, i16) of key tile kt holds exactly keys 16 kt
    // + 4 g .. +3 of row 16 rt + i16, i.e. half e / 4 = kt of its chunk; a
    // value lane (g, i16) reads the whole chunk (row tile, g, i16), which is
    // the P^T operand of k slots 8 g .. +7 (16 lanes read 256 contiguous
    // bytes).
    const uint32_t pw_off = (uint32_t)(rt * 1024 + g * 256 + i16 * 16 + kt * 8);
    const uint32_t pr_off = (uint32_t)(g * 256 + i16 * 16);
    // V^T operand of channel tile ct (channels 64 w + 16 ct .. +15), half tt:
    // lane (g, j4 = i16 / 4, a4 = i16 % 4) points at key 16 tt + 4 g + j4,
    // channels 64 w + 16 ct + 4 a4 .. +3: chunk 8 w + 2 ct + a4 / 2 at slot
    // (2 ct + a4 / 2) ^ (key % 8) of block (w, key / 8), byte 8 (a4 % 2); the
    // transposing read hands lane i16 channel i16 of those four keys, k slots
    // 8 g + 4 tt .. +3 of the P operand.
    uint32_t voff[2][4];
    {
        const int j4 = i16 >> 2, a4 = i16 & 3;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int key = 16 * tt + 4 * g + j4;
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4)
                voff[tt][c4] = (uint32_t)(w * (SK * 128) + (key >> 3) * 1024 + (key & 7) * 128 +
                                          (((2 * c4 + (a4 >> 1)) ^ (key & 7)) * 16) + (a4 & 1) * 8);
        }
    }

    f32x4 o[4][4];   // [channel tile][row tile]
    float mu = 0.f, l_part = 0.f, seen = -INFINITY;

    // S^T[key][row] of this wave's tile over the Dc + Dr channels, four K
    // operands in flight; keys past the split end are -inf.  When ld is
    // given, its loads go out one after every other MFMA.  With with_pv the
    // same pass accumulates O^T[d][row] += sum_key V[key][d] P[row][key] of
    // block pst (weights in buffer pb) for this wave's 64 channels and all 64
    // rows: its operands are read first and its 16 MFMAs sit between the
    // score steps, which they do not depend on.
    auto score = [&](int st, const Loads *ld, bool with_pv, int pst, int pb) {
        const char *kb = lds + (st % NB) * SB + koff;
        const char *kb1 = lds + (st % NB) * SB + (koff ^ 64u);
        auto kread = [&](int s) { return *(const bf16x8 *)((s & 1 ? kb1 : kb) + (s >> 1) * (SK * 128)); };
        // P^T and V^T operands of block pst, read before the score steps
        bf16x8 pr[4], vr[4];
        if (with_pv) {
            const uint32_t vb = (uint32_t)(uintptr_t)(const MLA_LDS void *)(lds + (pst % NB) * SB);
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4)
                pr[t4] = *(const bf16x8 *)(pbuf + pb * C::PB + t4 * 1024 + pr_off);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                struct {
                    i16x4 lo, hi;
                } pair{__builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4 *)(uintptr_t)(vb + voff[0][ct])),
                       __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4 *)(uintptr_t)(vb + voff[1][ct]))};
                vr[ct] = __builtin_bit_cast(bf16x8, pair);
            }
        }
        auto pv_step = [&](int ct, int t4) {
            if (with_pv && ct < 4)
                o[ct][t4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr[ct], pr[t4], o[ct][t4], 0, 0, 0);
        };
        f32x4 sc, sd;
        bf16x8 k0 = kread(0), k1 = kread(1), k2 = kread(2), k3 = kread(3);
#pragma unroll
        for (int s = 0; s < KS; s += 4) {
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qv[s], s ? sc : f32x4{}, 0, 0, 0);
            pv_step(s / 4, 0);
            if (s + 4 < KS)
                k0 = kread(s + 4);
            if (s + 1 < KS) {
                sd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qv[s + 1], s ? sd : f32x4{}, 0, 0, 0);
                if (s + 5 < KS)
                    k1 = kread(s + 5);
            }
            pv_step(s / 4, 1);
            if (ld && s / 2 < LA)
                load_one(*ld, s / 2);
            if (s + 2 < KS) {
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k2, qv[s + 2], sc, 0, 0, 0);
                if (s + 6 < KS)
                    k2 = kread(s + 6);
            }
            pv_step(s / 4, 2);
            if (s + 3 < KS) {
                sd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k3, qv[s + 3], sd, 0, 0, 0);
                if (s + 7 < KS)
                    k3 = kread(s + 7);
            }
            pv_step(s / 4, 3);
            if (ld && s / 2 + 1 < LA)
                load_one(*ld, s / 2 + 1);
        }
        sc += sd;
        const int lim = hi - (lo + st * SK) - 16 * kt - 4 * g;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            sc[r] = r < lim ? sc[r] : -INFINITY;
        return sc;
    };
    // row max of this wave's 16 keys (over the four lane groups), exchanged
    // with the other key tile through xrow[slot]; a workgroup barrier inside
    auto row_max_both = [&](float mx, int slot) {
        mx = mla_quad_max(mx);
        if (g == 0)
            xrow[slot][kt][rt * 16 + i16] = mx;
        __syncthreads();
        return fmaxf(mx, xrow[slot][kt ^ 1][rt * 16 + i16]);
    };
    // Wait until stage st has landed, given that the k stages after it have
    // been issued since (every stage but the last is full).  Only the loading
    // waves have loads outstanding.
    auto wait_stage = [&](int st, int k) {
        const bool two = k >= 2 && st + 2 < ns - 1, one = k >= 1 && st + 1 < ns - 1;
        if (w < 4) {
            if (two)
                mla_wait_vmcnt<2 * LA>();
            else if (one)
                mla_wait_vmcnt<LA>();
            else
                mla_wait_vmcnt<0>();
        } else {
            if (two)
                mla_wait_vmcnt<2 * LB>();
            else if (one)
                mla_wait_vmcnt<LB>();
            else
                mla_wait_vmcnt<0>();
        }
    };

    // bf16 weights of one block into weight buffer pb; their sum counts
    // toward the row sums unless the block is a repeat
    auto weights = [&](const f32x4 &sc, int pb, bool count) {
        typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
        bf16x4 pw;
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float pr = __builtin_amdgcn_exp2f(fmaf(sc[r], a.c, -mu));
            pw[r] = (__bf16)pr;
            sum += pr;
        }
        *(bf16x4 *)(pbuf + pb * C::PB + pw_off) = pw;
        l_part += count ? sum : 0.f;
    };

    // The weights are exp2(s c - mu) with mu fixed for a whole pass: the
    // first block's row max (over both key tiles) in the first pass.  Later
    // keys may exceed it; up to 2^64 the weights and their sums stay far
    // inside fp32 range and keep full relative precision.  When a row's max
    // passes mu + 64 the pass is repeated with mu = that row's max over the
    // split (then every weight is <= 1), so the accumulator is never
    // rescaled.  Block 0 is scored first; then per block u, after one
    // barrier (stage u + 1 has landed, the weights of block u are written,
    // and every wave is done with block u - 1, its stage and its weight
    // buffer) stage u + NBUF - 1 goes into the buffer of block u - 1, and
    // each wave scores block u + 1 into the other weight buffer while it
    // accumulates block u: the two MFMA streams are independent.  The last
    // trip scores its own block again (discarded), so the trip is one basic
    // block.
    static_assert(NBUF == 4, "three stages ahead");
    __shared__ int redo_flag;
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4)
                o[ct][t4] = f32x4{0.f, 0.f, 0.f, 0.f};
        l_part = 0.f;
        if constexpr (KV8) {
            // raw stages 0 and 1 issued, each widened as it lands and its slot
            // refilled at once (stages 2 and 3); then stage 2's chunks and
            // stage 4's pages are taken for the first trip
            pages8(0);
            issue8(0);
            pages8(1);
            issue8(1);
            take8(0);
            pages8(2);
            if (ns > 0)
                convert8(0);
            issue8(2);
            take8(1);
            pages8(3);
            if (1 < ns)
                convert8(1);
            issue8(3);
            take8(2);
            pages8(4);
        } else {
            for (int st = 0; st < NBUF - 1 && st < ns; ++st)
                issue(st);
        }
        if (ns > 0) {
            if constexpr (!KV8)
                wait_stage(0, ns - 1 < 2 ? ns - 1 : 2);
            __syncthreads();
            const f32x4 sc = score(0, nullptr, false, 0, 0);
            float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])) * a.c;
            if (pass == 0) {
                mx = row_max_both(mx, 0);
                mu = fabsf(mx) < INFINITY ? mx : 0.f;
            } else {
                mx = mla_quad_max(mx);
            }
            seen = fmaxf(seen, mx);
            weights(sc, 0, true);
        }
        for (int u = 0; u < ns; ++u) {
            if constexpr (!KV8) {
                if (u + 1 < ns)
                    wait_stage(u + 1, u + 2 < ns ? 1 : 0);
            }
            __syncthreads();
            const bool more = u + 1 < ns;
            Loads ld{};
            if constexpr (!KV8)
                ld = loads_of(u + NBUF - 1);
            if constexpr (KV8) {
                // stage u + 2 (taken at the end of the last trip) is widened
                // into the buffer of block u - 1, free since the barrier, and
                // its raw slot is refilled with stage u + 4; the next trip's
                // barrier publishes it
                if (u + 2 < ns)
                    convert8(u + 2);
                issue8(u + 4);
                // (kept apart from the score steps, whose operands fill the
                // registers)
                __builtin_amdgcn_sched_barrier(0);
            }
            const f32x4 sc = score(more ? u + 1 : u, KV8 ? nullptr : &ld, true, u, u & 1);
            const float mx = mla_quad_max(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])) * a.c);
            seen = fmaxf(seen, mx);
            weights(sc, (u + 1) & 1, more);
            if constexpr (KV8) {
                // for the next trip: stage u + 3's chunks, stage u + 5's pages
                take8(u + 3);
                pages8(u + 5);
            }
        }
        // repeat with the exact row max (over both key tiles) when some row
        // passed mu + 64; the decision is the workgroup's: the stages are shared
        const float seen_row = row_max_both(seen, 1);
        const bool need = __ballot(seen_row > mu + 64.f) != 0;
        if (tid == 0)
            redo_flag = 0;
        __syncthreads();
        if (need && lane == 0)
            redo_flag = 1;
        __syncthreads();
        if (pass == 1 || redo_flag == 0)
            break;
        mu = fabsf(seen_row) < INFINITY ? seen_row : 0.f;
        __syncthreads();    // every wave is done with the stages before they refill
    }

    // the row sums of both key tiles, and mu, for the value waves
    {
        const float lq = mla_quad_sum(l_part);
        if (g == 0) {
            xrow[2][kt][rt * 16 + i16] = lq;
            if (kt == 0)
                xrow[1][0][rt * 16 + i16] = mu;
        }
    }
    __syncthreads();
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
        const int mr = rg * 64 + t4 * 16 + i16;
        if (mr >= a.M)
            continue;
        const float lt = xrow[2][0][t4 * 16 + i16] + xrow[2][1][t4 * 16 + i16];
        const float mur = xrow[1][0][t4 * 16 + i16];
        const int r = mr / a.Hq, hh = mr % a.Hq;
        const int64_t row = ((int64_t)b * a.R + r) * a.Hq + hh;
        const float inv = lt != 0.f ? 1.f / lt : 0.f;
        float *dst = a.ws_o + (row * a.n_split + split) * 512 + 64 * w + 4 * g;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
            *(float4 *)(dst + 16 * ct) = make_float4(o[ct][t4][0] * inv, o[ct][t4][1] * inv,
                                                     o[ct][t4][2] * inv, o[ct][t4][3] * inv);
        if (w == 0 && g == 0)
            a.ws_lse[row * a.n_split + split] = lt != 0.f ? mur + __log2f(lt) : -INFINITY;
    }
}

// Window part and merge: one wave per (request b, row r, head h).  The
// window keys are the set bits j < W of the row's mask at logical position
// P + j; lane l holds channels 8 l .. 8 l + 7 of the latent part (and, for
// l < Dr / 8, rotary channels 8 l .. +7).  Lane j looks up the latent row of
// window key j (all page lookups at once); the keys are then taken eight at
// a time with their row loads in flight together, with an online softmax
// over the groups.  Then the merge with the n_split prefix partials (their
// lse2 read at once, one per lane): lse2 = log2 sum_k 2^lse2_k, out = sum_k
// 2^(lse2_k - lse2) o_k.
template <int DR, bool KV8>
__global__ void __launch_bounds__(256) k_mla_window_merge(MlaArgs a) {
    constexpr int DK = 512 + DR;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= (int64_t)a.B * a.R * a.Hq)
        return;
    const int r = (int)((row / a.Hq) % a.R);
    const int b = (int)(row / ((int64_t)a.Hq * a.R));
    int P = a.prefix_len[b];
    P = P < 0 ? 0 : (P > a.max_prefix_len ? a.max_prefix_len : P);
    auto widen = [](const int4 x, float (&f)[8]) {
        const uint32_t u[4] = {(uint32_t)x.x, (uint32_t)x.y, (uint32_t)x.z, (uint32_t)x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[2 * e] = __uint_as_float(u[e] << 16);
            f[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
        }
    };
    const uint16_t *qp = a.q + row * DK;
    // the query stays packed (bf16) and is widened per key: fewer registers,
    // more waves in flight.  Under an FP8 latent cache it is the E4M3 query
    // (rounded, held as bf16) for window keys too.
    int4 qcp = *(const int4 *)(qp + 8 * lane);
    int4 qrp = DR > 0 && lane < DR / 8 ? *(const int4 *)(qp + 512 + 8 * lane) : make_int4(0, 0, 0, 0);
    if constexpr (KV8) {
        qcp = mla_bf16x8_round_e4m3(qcp);
        qrp = mla_bf16x8_round_e4m3(qrp);
    }
    // a latent row's 8 channels of this lane as packed bf16 (FP8 rows widened)
    auto load8 = [&](int64_t ro, int ch) {
        if constexpr (KV8) {
            const int2 x = *(const int2 *)((const uint8_t *)a.lat + ro + ch);
            int4 lo, hi;
            mla_fp8x16_to_bf16(make_int4(x.x, x.y, 0, 0), lo, hi);
            return lo;
        } else {
            return *(const int4 *)(a.lat + ro + ch);
        }
    };

    uint64_t bits = a.masks[(int64_t)b * a.R + r];
    if (a.W < 64)
        bits &= (1ull << a.W) - 1;
    // the latent row of window key `lane` (keys whose page falls outside the
    // table are dropped from the set)
    const int ps = 1 << a.ps_shift;
    int64_t myrow = 0;
    {
        const int t = P + lane;
        const int lp = t >> a.ps_shift;
        const bool set = (bits >> lane) & 1;
        if (set && lp < a.max_pages) {
            int64_t pg = a.page_table[(int64_t)b * a.max_pages + lp];
            pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
            myrow = pg * a.stride_page + (int64_t)(t & (ps - 1)) * a.stride_token;
        }
        bits &= __ballot(set && lp < a.max_pages);
    }
    float mw = -INFINITY, lw = 0.f, ow[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        ow[e] = 0.f;
    while (bits) {
        constexpr int GK = 8;
        int js[GK];
        int n = 0;
#pragma unroll
        for (int i = 0; i < GK; ++i) {
            js[i] = bits ? __builtin_ctzll(bits) : -1;
            if (bits) {
                bits &= bits - 1;
                ++n;
            }
        }
        int4 xk[GK], xr[GK];
#pragma unroll
        for (int i = 0; i < GK; ++i) {
            xk[i] = xr[i] = make_int4(0, 0, 0, 0);
            if (js[i] >= 0) {
                const int64_t ro = ((int64_t)__builtin_amdgcn_readlane((int)(myrow >> 32), js[i]) << 32) |
                                   (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)myrow, js[i]);
                xk[i] = load8(ro, 8 * lane);
                if (DR > 0 && lane < DR / 8)
                    xr[i] = load8(ro, 512 + 8 * lane);
            }
        }
        float sj[GK];
#pragma unroll
        for (int i = 0; i < GK; ++i) {
            float kv[8], rv[8], qc[8], qr[8];
            widen(xk[i], kv);
            widen(xr[i], rv);
            widen(qcp, qc);
            widen(qrp, qr);
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                d = fmaf(qc[e], kv[e], d);
            if (DR > 0) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    d = fmaf(qr[e], rv[e], d);
            }
            sj[i] = d;
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
            for (int i = 0; i < GK; ++i)
                sj[i] += __shfl_xor(sj[i], o);
        float mg = mw;
#pragma unroll
        for (int i = 0; i < GK; ++i) {
            sj[i] *= a.c;    // exp2 domain
            if (i < n)
                mg = fmaxf(mg, sj[i]);
        }
        // (equal maxima, both -inf included, leave the running sums as they are)
        const float alpha = mw == mg ? 1.f : __builtin_amdgcn_exp2f(mw - mg);
        lw *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            ow[e] *= alpha;
#pragma unroll
        for (int i = 0; i < GK; ++i) {
            if (i < n) {
                float kv[8];
                widen(xk[i], kv);
                const float pj = sj[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sj[i] - mg);
                lw += pj;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    ow[e] = fmaf(pj, kv[e], ow[e]);
            }
        }
        mw = mg;
    }
    // merge: the window part (o = ow / lw, lse2 = mw + log2 lw) and the
    // prefix partials; lane k reads the lse2 of split k
    const float lse_w = lw != 0.f ? mw + __log2f(lw) : -INFINITY;
    float mx = lse_w;
    for (int k0 = 0; k0 < a.n_split; k0 += 64) {
        const float l = k0 + lane < a.n_split ? a.ws_lse[row * a.n_split + k0 + lane] : -INFINITY;
        float lm = l;
        bool nan = l != l;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            lm = fmaxf(lm, __shfl_xor(lm, o));
        nan = __ballot(nan) != 0;
        mx = (nan || mx != mx) ? NAN : fmaxf(mx, lm);
    }
    float acc[8], z = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc[e] = 0.f;
    if (mx != -INFINITY) {
        if (lse_w != -INFINITY) {
            const float zw = __builtin_amdgcn_exp2f(lse_w - mx);
            const float inv = 1.f / lw;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[e] = zw * ow[e] * inv;
            z = zw;
        }
        for (int k0 = 0; k0 < a.n_split; k0 += 64) {
            const float l = k0 + lane < a.n_split ? a.ws_lse[row * a.n_split + k0 + lane] : -INFINITY;
            // a split without keys (lse2 = -inf) is skipped, marked by -1
            const float zl = l == -INFINITY ? -1.f : __builtin_amdgcn_exp2f(l - mx);
            const int kn = a.n_split - k0 < 64 ? a.n_split - k0 : 64;
            int k = 0;
            for (; k + 2 <= kn; k += 2) {
                float4 p[2][2];
                float zk[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    zk[i] = __shfl(zl, k + i);
                    const float4 *src = (const float4 *)(a.ws_o + (row * a.n_split + k0 + k + i) * 512 + 8 * lane);
                    p[i][0] = src[0];
                    p[i][1] = src[1];
                }
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    if (zk[i] < 0.f)
                        continue;
                    acc[0] = fmaf(zk[i], p[i][0].x, acc[0]);
                    acc[1] = fmaf(zk[i], p[i][0].y, acc[1]);
                    acc[2] = fmaf(zk[i], p[i][0].z, acc[2]);
                    acc[3] = fmaf(zk[i], p[i][0].w, acc[3]);
                    acc[4] = fmaf(zk[i], p[i][1].x, acc[4]);
                    acc[5] = fmaf(zk[i], p[i][1].y, acc[5]);
                    acc[6] = fmaf(zk[i], p[i][1].z, acc[6]);
                    acc[7] = fmaf(zk[i], p[i][1].w, acc[7]);
                    z += zk[i];
                }
            }
            for (; k < kn; ++k) {
                const float zk = __shfl(zl, k);
                if (zk < 0.f)
                    continue;
                const float4 *src = (const float4 *)(a.ws_o + (row * a.n_split + k0 + k) * 512 + 8 * lane);
                const float4 p0 = src[0], p1 = src[1];
                acc[0] = fmaf(zk, p0.x, acc[0]);
                acc[1] = fmaf(zk, p0.y, acc[1]);
                acc[2] = fmaf(zk, p0.z, acc[2]);
                acc[3] = fmaf(zk, p0.w, acc[3]);
                acc[4] = fmaf(zk, p1.x, acc[4]);
                acc[5] = fmaf(zk, p1.y, acc[5]);
                acc[6] = fmaf(zk, p1.z, acc[6]);
                acc[7] = fmaf(zk, p1.w, acc[7]);
                z += zk;
            }
        }
    }
    const float invz = z != 0.f ? 1.f / z : 0.f;
    uint32_t packed[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        packed[e] = (uint32_t)mla_bf16_bits(acc[2 * e] * invz) |
                    ((uint32_t)mla_bf16_bits(acc[2 * e + 1] * invz) << 16);
    *(int4 *)(a.out + row * 512 + 8 * lane) =
        make_int4((int)packed[0], (int)packed[1], (int)packed[2], (int)packed[3]);
    if (a.lse2 && lane == 0)
        a.lse2[row] = mx == -INFINITY ? -INFINITY : mx + __log2f(z);
}

struct MlaPlan {
    int RG, n_split, kps;
    size_t o_bytes, bytes;
};

inline size_t mla_align256(size_t x) { return (x + 255) & ~size_t(255); }

MlaPlan mla_plan(int B, int R, int Hq, int max_prefix_len, int page_size) {
    MlaPlan p{};
    const long long M = (long long)R * Hq;
    p.RG = (int)((M + 63) / 64);
    const long long base = (long long)B * p.RG;
    int n = base > 0 ? (int)((256 + base - 1) / base) : 1;
    const int by_keys = max_prefix_len / 128;            // >= 4 stages per split
    n = n < by_keys ? n : by_keys;
    n = n < 1 ? 1 : n;
    // a multiple of 8 (request, split) streams keeps the eight XCDs equally
    // busy (each stream lives on one XCD); take one if it costs at most twice
    // the splits
    for (int m = n; m <= 2 * n && m <= by_keys; ++m)
        if (((long long)B * m) % 8 == 0) {
            n = m;
            break;
        }
    int kps;
    for (;;) {
        kps = (max_prefix_len + n - 1) / n;
        kps = ((kps + 31) / 32) * 32;
        if (kps < 32)
            kps = 32;
        if ((long long)kps / page_size + 2 <= kMlaPt)
            break;
        ++n;
    }
    p.kps = kps;
    p.n_split = max_prefix_len > 0 ? (max_prefix_len + kps - 1) / kps : 1;
    const long long rows = (long long)B * R * Hq;
    p.o_bytes = mla_align256((size_t)rows * p.n_split * 512 * sizeof(float));
    p.bytes = p.o_bytes + mla_align256((size_t)rows * p.n_split * sizeof(float));
    return p;
}

inline hipStream_t MS(void *s) { return (hipStream_t)s; }

}  // namespace

using tav::Checks;
using tav::str;

extern "C" size_t tree_attention_mla_workspace_size(int32_t B, int32_t R, int32_t Hq, int32_t Dc,
                                                    int32_t Dr, int32_t max_prefix_len,
                                                    int32_t page_size) {
    if (B < 0 || R < 1 || R > 64 || Hq < 1 || Dc != 512 || (Dr != 0 && Dr != 64) ||
        max_prefix_len < 0 || !tav::is_pow2(page_size) || page_size > 1024)
        return 0;
    return mla_plan(B, R, Hq, max_prefix_len, page_size).bytes;
}

extern "C" tav_status tree_attention_mla(const void *q, const void *latent, tav_dtype dtype,
                                         int64_t stride_page, int64_t stride_token,
                                         int64_t num_pages, const int32_t *page_table,
                                         int32_t max_pages, int32_t page_size,
                                         const int32_t *prefix_len, int32_t max_prefix_len,
                                         const uint64_t *masks, int32_t W, int32_t B, int32_t R,
                                         int32_t Hq, int32_t Dc, int32_t Dr, float sm_scale,
                                         void *out, float *lse2, void *workspace,
                                         size_t workspace_bytes, void *stream) {
    Checks c;
    TAV_NEED(c, B >= 0, TAV_ERR_INVALID_ARG, "B must be >= 0, got " + str(B));
    TAV_NEED(c, R >= 1 && R <= 64, TAV_ERR_INVALID_ARG, "R must be in [1, 64], got " + str(R));
    TAV_NEED(c, W >= 0 && W <= 64, TAV_ERR_INVALID_ARG, "W must be in [0, 64], got " + str(W));
    TAV_NEED(c, Hq >= 1, TAV_ERR_INVALID_ARG, "Hq must be >= 1, got " + str(Hq));
    TAV_NEED(c, Dc == 512, TAV_ERR_UNSUPPORTED, "Dc (kv_lora_rank) must be 512, got " + str(Dc));
    TAV_NEED(c, Dr == 0 || Dr == 64, TAV_ERR_UNSUPPORTED, "Dr must be 0 or 64, got " + str(Dr));
    TAV_NEED(c, dtype == TAV_BF16 || dtype == TAV_FP8_E4M3, TAV_ERR_UNSUPPORTED,
             "the latent cache must be TAV_BF16 or TAV_FP8_E4M3 (bf16 query), got " + str(dtype));
    const int64_t elem = dtype == TAV_FP8_E4M3 ? 1 : 2;
    TAV_NEED(c, tav::is_pow2(page_size) && page_size <= 1024, TAV_ERR_UNSUPPORTED,
             "page_size must be a power of two <= 1024, got " + str(page_size));
    TAV_NEED(c, max_prefix_len >= 0, TAV_ERR_INVALID_ARG, "max_prefix_len must be >= 0");
    TAV_NEED(c, max_pages >= 1 && (long long)max_pages * page_size >= (long long)max_prefix_len + W,
             TAV_ERR_INVALID_ARG, "max_pages * page_size must cover max_prefix_len + W");
    TAV_NEED(c, num_pages >= 1, TAV_ERR_INVALID_ARG, "num_pages must be >= 1");
    TAV_NEED(c, stride_token >= Dc + Dr && (stride_token * elem) % 16 == 0 &&
                 (stride_page * elem) % 16 == 0,
             TAV_ERR_UNSUPPORTED,
             "latent rows must hold Dc + Dr contiguous elements at 16-byte aligned strides");
    TAV_NEED(c, std::isfinite(sm_scale), TAV_ERR_INVALID_ARG, "sm_scale must be finite");
    if (B > 0) {
        TAV_NEED(c, q && latent && page_table && prefix_len && masks && out, TAV_ERR_INVALID_ARG,
                 "q, latent, page_table, prefix_len, masks and out must be set");
        TAV_NEED(c, (((uintptr_t)q | (uintptr_t)latent | (uintptr_t)out) & 15) == 0,
                 TAV_ERR_INVALID_ARG, "q, latent and out must be 16-byte aligned");
        if (c.status == TAV_OK) {
            const MlaPlan p = mla_plan(B, R, Hq, max_prefix_len, page_size);
            TAV_NEED(c, workspace && ((uintptr_t)workspace & 255) == 0, TAV_ERR_WORKSPACE,
                     "workspace must be set and 256-byte aligned");
            TAV_NEED(c, workspace_bytes >= p.bytes, TAV_ERR_WORKSPACE,
                     "workspace has " + str((long long)workspace_bytes) + " bytes, needs " +
                         str((long long)p.bytes));
        }
    }
    if (c.status != TAV_OK || B == 0)
        return tav::finish("tree_attention_mla", c);
    const MlaPlan p = mla_plan(B, R, Hq, max_prefix_len, page_size);
    MlaArgs a{};
    a.q = (const uint16_t *)q;
    a.lat = (const uint16_t *)latent;   // byte addressed under an FP8 cache
    a.stride_page = stride_page;
    a.stride_token = stride_token;
    a.num_pages = num_pages;
    a.page_table = page_table;
    a.max_pages = max_pages;
    a.ps_shift = tav::ilog2(page_size);
    a.prefix_len = prefix_len;
    a.max_prefix_len = max_prefix_len;
    a.masks = masks;
    a.W = W;
    a.B = B;
    a.R = R;
    a.Hq = Hq;
    a.M = R * Hq;
    a.RG = p.RG;
    a.n_split = p.n_split;
    a.kps = p.kps;
    const float scale = sm_scale > 0.f ? sm_scale : 1.f / std::sqrt((float)(Dc + Dr));
    a.c = scale * kLog2eM;
    a.ws_o = (float *)workspace;
    a.ws_lse = (float *)((char *)workspace + p.o_bytes);
    a.out = (uint16_t *)out;
    a.lse2 = lse2;
    if (max_prefix_len > 0) {
        const long long streams = (long long)B * p.n_split;
        const unsigned grid = (unsigned)(((streams + 7) / 8) * 8 * p.RG);
        const bool kv8 = dtype == TAV_FP8_E4M3;
        if (Dr == 64 && kv8)
            hipLaunchKernelGGL((k_mla_prefix<64, true>), dim3(grid), dim3(512), 0, MS(stream), a);
        else if (Dr == 64)
            hipLaunchKernelGGL((k_mla_prefix<64, false>), dim3(grid), dim3(512), 0, MS(stream), a);
        else if (kv8)
            hipLaunchKernelGGL((k_mla_prefix<0, true>), dim3(grid), dim3(512), 0, MS(stream), a);
        else
            hipLaunchKernelGGL((k_mla_prefix<0, false>), dim3(grid), dim3(512), 0, MS(stream), a);
        tav_status st = tav::launched("tree_attention_mla");
        if (st != TAV_OK)
            return st;
    } else {
        a.n_split = 0;
    }
    const long long rows = (long long)B * R * Hq;
    const dim3 wgrid((unsigned)((rows + 3) / 4));
    if (Dr == 64 && dtype == TAV_FP8_E4M3)
        hipLaunchKernelGGL((k_mla_window_merge<64, true>), wgrid, dim3(256), 0, MS(stream), a);
    else if (Dr == 64)
        hipLaunchKernelGGL((k_mla_window_merge<64, false>), wgrid, dim3(256), 0, MS(stream), a);
    else if (dtype == TAV_FP8_E4M3)
        hipLaunchKernelGGL((k_mla_window_merge<0, true>), wgrid, dim3(256), 0, MS(stream), a);
    else
        hipLaunchKernelGGL((k_mla_window_merge<0, false>), wgrid, dim3(256), 0, MS(stream), a);
    return tav::launched("tree_attention_mla");
}
