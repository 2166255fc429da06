// tree_attention: split-K paged prefix decode + masked tree window + base-2
// LSE merge, for gfx950 (CDNA4).
//
// The cascade follows "Draft-tree speculation", section "One tree attention:
// the leaf's decode for the prefix, a small kernel for the tree": a query
// row attends to all of the committed prefix, its uint64 ancestor mask only
// chooses among the W window keys, and the two partial results are combined
// by their base-2 log-sum-exp.  "EAGLE Tree Attention candidate layout,
// positions and visibility", section 4, describes the same split: a prefix
// shared by every query, a suffix filtered per query, and a merge that
// weights each part's normalised output by its softmax mass.
//
// Kernels:
//   k_prefix_mfma<D, NRB, NKS, KV8>  bf16 (or FP8 E4M3 K/V).  One workgroup of
//       NRB x NKS waves per (request, kv head, row group, split).  All R x
//       (Hq/Hkv) query rows of a kv head are folded into the MFMA N
//       dimension, so one pass over a K/V page serves every row and head of
//       the group.  Pages stream HBM -> LDS with direct-to-LDS 16-byte loads,
//       NBUF stages deep; S^T = K Q^T and O^T = V^T P^T run on
//       v_mfma_f32_32x32x16_bf16 with fp32 accumulation; softmax is online in
//       the exp2 domain.  Writes one (O, lse2) partial per split (its NKS key
//       subsets combined in LDS); with one row block over bf16 K/V run as a
//       single split, it also takes the window keys as one more stage and
//       writes the output itself.
//   k_prefix_mfma_pipe  the software-pipelined kernel for 256 folded rows.
//       Run as a single split over bf16 K/V, with the masks and the output
//       given, it also takes the window keys as one more stage and writes
//       the output itself (no window or merge launch).
//   k_prefix_f32<D>  fp32 inputs, vector ALU, one wave per (row, split).
//   k_window_mfma  bf16: one tile of window keys per kv head serves all its
//       rows on MFMA, the masks applied in-kernel; writes the window partial
//       (or, with a single prefix partial, merges the row itself).
//   k_merge  bf16: one wave per (request, row, head), or 4 or 8 waves per
//       row with many splits, merges every partial through its base-2 LSE
//       into out / lse2.
//   k_window_merge  fp32: one wave per (request, row, head): the masked window
//       keys (popcount(mask) of them, never the unseen ones) and the merge of
//       every prefix partial with the window part into out / lse2.
#include <cmath>
#include <mutex>
#include <type_traits>
#include <utility>

#include "tav_internal.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kPtMax = 2560;        // page-table entries one split may span
constexpr int kLdsStageBudget = 144 * 1024;
constexpr int kPipeStageKeys = 64;   // keys per stage of the pipelined kernel (32 or 64)

__device__ inline float bf16_bits_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ inline uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ inline float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        x += __shfl_xor(x, o);
    return x;
}

__device__ inline float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

// A softmax part with denominator l has keys unless l == 0.  A NaN l (a NaN
// score or value among visible keys) is kept, so it reaches the output as the
// definition's arithmetic would carry it; only l == 0 means "no key".
__device__ inline bool has_keys(float l) { return !(l == 0.f); }

// exp2 with exp2(-inf) = 0 (the hardware instruction handles it).
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Direct-to-LDS 16-byte load (global_load_lds_dwordx4): lane i's 16 bytes at
// `src` land at LDS byte address lds_base + 16 i.  It is issued as inline
// assembly so that the compiler does not track it as an LDS write: otherwise
// its wait insertion makes LDS reads it cannot attribute to one buffer wait
// for every such load in flight (vmcnt(0)), which would serialise the stage
// pipeline.  Completion is established explicitly: wait_vmcnt<N>() for the
// issuing wave, then a workgroup barrier.  lds_base must be wave-uniform.
// Pages are read once per call, so the loads carry the non-temporal hint:
// streaming them past the caches costs less energy per byte, and the chip
// runs this kernel at its board power limit.
__device__ __forceinline__ void dma_load16(const void *src, uint32_t lds_base) {
    int m0v;   // m0 is an output, so the compiler keeps no value of its own there
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
                 : "={m0}"(m0v)
                 : "v"(src), "s"(lds_base)
                 : "memory");
}

// Direct-to-LDS 16-byte load with a wave-uniform 64-bit base and a per-lane
// 32-bit byte offset; lane i's 16 bytes land at LDS byte lds_base + 16 i.
// Completion is tracked as for dma_load16.
__device__ __forceinline__ void dma_load16_s(const void *base, uint32_t voff, uint32_t lds_base) {
    int m0v;   // m0 is an output, so the compiler keeps no value of its own there
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 : "={m0}"(m0v)
                 : "v"(voff), "s"(base), "s"(lds_base)
                 : "memory");
}

// 16 FP8 E4M3 values (one 16-byte chunk) -> 16 bf16 values (two chunks);
// the conversion is exact (every E4M3 value, NaN included, is a bf16 value).
__device__ __forceinline__ void fp8x16_to_bf16(const int4 x, int4 &lo, int4 &hi) {
    auto c0 = [](int w) {
        return __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w, 1.0f, false));
    };
    auto c1 = [](int w) {
        return __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w, 1.0f, true));
    };
    lo = make_int4(c0(x.x), c1(x.x), c0(x.y), c1(x.y));
    hi = make_int4(c0(x.z), c1(x.z), c0(x.w), c1(x.w));
}

// x rounded to the nearest FP8 E4M3 value (ties to even), as fp32; magnitudes
// past the largest finite value (448) give +-448 and NaN stays NaN.  Above
// the subnormal range an E4M3 value has 4 significant bits, so the quantum
// at binary exponent e is 2^(e - 3); below 2^-6 it is 2^-9.  Scaling by
// those powers of two is exact and v_rndne_f32 rounds ties to even.
__device__ inline float round_e4m3(float x) {
    if (!(fabsf(x) <= 448.f))
        return x != x ? x : copysignf(448.f, x);
    const float a = fabsf(x);
    int e = (int)((__float_as_uint(a) >> 23) & 0xff) - 127;
    e = e < -6 ? -6 : e;
    const float up = __uint_as_float((uint32_t)(3 - e + 127) << 23);     // 2^(3 - e)
    const float dn = __uint_as_float((uint32_t)(e - 3 + 127) << 23);     // 2^(e - 3)
    return copysignf(__builtin_rintf(a * up) * dn, x);
}

// The query operand of the prefix under an FP8 cache: each bf16 value rounded
// to E4M3 (held as bf16, which represents every E4M3 value exactly).  The
// products with E4M3 keys are then exact, as in an FP8 matrix product.
__device__ inline bf16x8 bf16x8_round_e4m3(bf16x8 v) {
    // element access through a whole-vector cast: a bit cast of a single
    // subscripted element reads element 0 whatever the index
    typedef __attribute__((__vector_size__(8 * sizeof(uint16_t)))) uint16_t u16x8;
    const u16x8 u = __builtin_bit_cast(u16x8, v);
    u16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        r[i] = f32_to_bf16_bits(round_e4m3(bf16_bits_to_f32(u[i])));
    return __builtin_bit_cast(bf16x8, r);
}

// fp32 value of one FP8 E4M3 code
__device__ __forceinline__ float fp8_to_f32(uint8_t b) {
    const int w = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)b, 1.0f, false));
    return __uint_as_float((uint32_t)w << 16);
}

__device__ __forceinline__ uint32_t lds_off(const void *p) {
    return (uint32_t)(uintptr_t)(const LDS_AS void *)p;
}

// Combine lane l with lane l ^ 32 on the vector ALU (v_permlane32_swap):
// after swapping a copy, one result holds the lower-half value of the pair and
// the other the upper-half value.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(std::forward<F>(f));
    }
}

// s_waitcnt vmcnt(N) without waiting on LGKM / EXP counters (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14).
template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Completes a value loaded from memory where it is called.  The compiler
// otherwise places the wait for the load before the value's first use,
// which inside a pipelined loop (with its state merged over the back edge)
// becomes a wait for every outstanding load, the in-flight stages included.
template <typename T>
__device__ __forceinline__ void settle(T &x) {
    asm volatile("" : "+v"(x));
}

struct PrefixArgs {
    const void *q;
    const void *k;
    const void *v;
    int64_t stride_page, stride_head, stride_token, num_pages;
    const int32_t *page_table;
    int32_t max_pages, ps_shift;
    const int32_t *prefix_len;
    int32_t max_prefix_len, prefix_window;
    int32_t B, R, Hq, Hkv, G, M, RG, n_split, kps, S;
    float c;  // sm_scale * log2(e): scores in the exp2 domain
    float *ws_o;
    float *ws_lse;
    // a single split on the pipelined kernel over bf16 K/V, with the masks
    // and output given: the split also attends the window keys under the
    // masks and writes the output itself (no window or merge launch)
    int32_t fuse, W;
    const uint64_t *masks;
    void *out;
    float *lse2;
};

// Visible prefix range [lo, hi) of split `split` of request b.
struct KeyRange {
    int lo, hi;
};
__device__ inline KeyRange split_range(const PrefixArgs &a, int b, int split) {
    int P = a.prefix_len[b];
    P = P < 0 ? 0 : (P > a.max_prefix_len ? a.max_prefix_len : P);
    const int p_lo = (a.prefix_window > 0 && P > a.prefix_window) ? P - a.prefix_window : 0;
    const int lo = p_lo + split * a.kps;
    int hi = lo + a.kps;
    hi = hi < P ? hi : P;
    return {lo, hi < lo ? lo : hi};
}

__device__ inline int64_t clamp_page(int64_t p, int64_t n) { return p < 0 ? 0 : (p >= n ? n - 1 : p); }

// XOR swizzle of the 16-byte chunks of a key row in LDS.  It makes both LDS
// read patterns conflict-free: the K operand (lanes = 32 keys, one chunk) and
// the transposing V reads (16-lane groups = 4 keys x 32 bytes).
template <int D>
__device__ inline int swz(int key) {
    const int x = ((key & 3) << 1) | ((key >> 2) & 1);
    return D == 128 ? (x | (key & 8)) : x;
}

template <int D, int NRB, int NKS>
struct MfmaCfg {
    static constexpr int WAVES = NRB * NKS;       // waves per workgroup
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int SK = 32 * NKS;           // keys per stage
    static constexpr int CH = D / 8;              // 16-byte chunks per key row
    static constexpr int ROWB = D * 2;            // bytes per key row (bf16)
    static constexpr int SB = SK * ROWB * 2;      // stage bytes, K then V
    static constexpr int NBUF0 = (WAVES <= 2 ? 64 * 1024 : kLdsStageBudget) / SB;   // two 2-wave workgroups share a CU
    static constexpr int NBUF = NBUF0 > 8 ? 8 : NBUF0;
    static constexpr int LPS = SB / (THREADS * 16);   // 16-byte loads per thread per stage
    static_assert(NBUF >= 2, "stage too large");
    static_assert(LPS >= 1 && SB % (THREADS * 16) == 0, "stage split");
    static_assert((NBUF - 2) * LPS < 64, "vmcnt range");
};

// Split-K paged prefix decode on MFMA.  One workgroup = WAVES waves = NRB row
// blocks of 32 folded query rows x NKS key subsets; every wave owns 32 rows
// and, per stage, one 32-key block.  With 8 waves a SIMD holds two waves, so
// one wave's MFMAs overlap the other's softmax; a 2-wave workgroup (bf16, at
// most 32 rows) keeps two 32 KB stages, so that two workgroups share a CU and
// one's prologue and epilogue overlap the other's stream.
template <int D, int NRB, int NKS, bool KV8>
__global__ void __launch_bounds__(64 * NRB * NKS, 1) k_prefix_mfma(PrefixArgs a) {
    using C = MfmaCfg<D, NRB, NKS>;
    constexpr int SK = C::SK, CH = C::CH, ROWB = C::ROWB, SB = C::SB, NBUF = C::NBUF,
                  LPS = C::LPS, THREADS = C::THREADS;
    constexpr int ROWS_WG = NRB * 32;
    constexpr int KSTEPS = D / 16;
    constexpr int DT = D / 32;                    // 32-wide d tiles
    // FP8 rows of 128 channels are staged raw by direct-to-LDS loads: a stage
    // is SK rows of K, then SK rows of V, D bytes each
    // (a 4-wave workgroup keeps two raw stages, 64 KB, so that two workgroups
    // share a CU and each SIMD runs two waves; wider workgroups fill the CU
    // alone and keep up to eight)
    constexpr bool KVD = KV8 && D == 128;
    constexpr int SB8 = SK * D * 2;
    constexpr int NB8A = (THREADS <= 256 ? 64 * 1024 : kLdsStageBudget) / SB8;
    constexpr int NBUF8 = NB8A > 8 ? 8 : NB8A;
    constexpr int LPS8 = SB8 / (THREADS * 16);    // 16-byte loads per thread per raw stage
    static_assert(!KVD || (NBUF8 >= 2 && LPS8 >= 1 && SB8 % (THREADS * 16) == 0 &&
                           (NBUF8 - 2) * LPS8 < 64), "fp8 stage split");
    constexpr int LDSB = KVD ? NBUF8 * SB8 : NBUF * SB;

    __shared__ __attribute__((aligned(16))) char lds[LDSB];
    __shared__ int32_t pt[kPtMax];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane >> 5;  // lane half
    const int l32 = lane & 31;

    // Work unit.  Workgroups are dispatched round-robin over the 8 XCDs; the
    // row groups of one (request, kv head, split) read the same pages, so
    // they are kept on one XCD (one L2) when the unit count allows it.
    const int units = a.B * a.Hkv * a.n_split;
    int rg, unit;
    const int id = blockIdx.x;
    if (a.RG > 1 && (units & 7) == 0) {
        const int xcd = id & 7, slot = id >> 3;
        rg = slot % a.RG;
        unit = (slot / a.RG) * 8 + xcd;
    } else {
        rg = id % a.RG;
        unit = id / a.RG;
    }
    const int split = unit % a.n_split;
    const int g = (unit / a.n_split) % a.Hkv;
    const int b = unit / (a.n_split * a.Hkv);

    const KeyRange kr = split_range(a, b, split);
    // With pages of 8 or more keys the keys of one load instruction (64 / CH
    // consecutive keys) share a page, so loads take a wave-uniform page base;
    // stages then start at the 8-key boundary at or below the split start and
    // keys outside [lo, hi) are neither loaded nor visible.
    const bool wave_pages = (!KV8 || KVD) && a.ps_shift >= 3;
    const int kb0 = wave_pages ? (kr.lo & ~7) : kr.lo;
    const int nkeys = kr.hi > kr.lo ? kr.hi - kb0 : 0;
    const int ns = (nkeys + SK - 1) / SK;
    const int rbw = w % NRB;   // this wave's row block
    const int ks = w / NRB;    // this wave's key subset within a stage
    const int rows_base = rg * ROWS_WG + rbw * 32;

    // A fused launch (one row block, bf16 K/V, one split, whose range ends
    // at the prefix length P): the window keys P .. P + W - 1 are one more
    // stage, and the page-table slice also covers their pages.
    constexpr bool FUSE = !KV8 && NRB == 1;
    int Pw = 0;
    const bool wown = FUSE && a.fuse && a.W > 0;
    if (wown) {
        Pw = a.prefix_len[b];
        Pw = Pw < 0 ? 0 : (Pw > a.max_prefix_len ? a.max_prefix_len : Pw);
    }
    __shared__ uint32_t wbad[2];   // window keys 0..31, 32..63 with a non-finite V value
    __shared__ uint64_t wmk[FUSE ? 32 : 1];
    if (tid < 2)
        wbad[tid] = 0u;
    if (wown && tid < 32) {
        const int mm = rows_base + tid;
        wmk[tid] = mm < a.M ? a.masks[(int64_t)b * a.R + mm / a.G] : 0ull;
    }

    // page-table slice of this split: its entries are loaded into registers
    // first, the query loads go out behind them, and the entries are stored
    // to LDS after (so the stores wait for the table loads only, and the two
    // round trips overlap)
    const bool any_pt = nkeys > 0 || wown;
    const int lp0 = any_pt ? ((nkeys > 0 ? kb0 : Pw) >> a.ps_shift) : 0;
    const int npt = any_pt ? (((wown ? Pw + a.W : kr.hi) - 1) >> a.ps_shift) - lp0 + 1 : 0;
    constexpr int PTPT = (kPtMax + THREADS - 1) / THREADS;   // entries per thread, at most
    int64_t ptv[PTPT];
#pragma unroll
    for (int j = 0; j < PTPT; ++j) {
        const int i = tid + j * THREADS;
        ptv[j] = i < npt && i < kPtMax ? a.page_table[(int64_t)b * a.max_pages + lp0 + i] : 0;
    }
    // zero the stage buffers once: the last, partial stage leaves rows unloaded
    // and they must hold finite values (their softmax weight is exactly 0)
    for (int i = tid; i < LDSB / 16; i += THREADS)
        reinterpret_cast<int4 *>(lds)[i] = make_int4(0, 0, 0, 0);

    // Q^T operand in registers, bf16: lane (row n = l32, half hl) holds 8
    // channels of Q[row] per 16-channel k step.  Under an FP8 cache the query
    // is rounded to E4M3 (held as bf16, which holds every E4M3 value), so the
    // bf16 products with the widened E4M3 keys are exact and accumulate in
    // fp32.  (The FP8 MFMAs are not used for the scores: they sum each
    // 64-product group at about 12 bits relative to its largest product.)
    // Steps take channels 16 kk + 8 hl .. +8, except for FP8 rows of 128
    // channels, whose K operand lane reads whole 16-byte E4M3 chunks 4 c +
    // 2 hl + e (c, e = 0, 1): step 4 c + 2 e + h then takes channels
    // 16 (4 c + 2 hl + e) + 8 h .. +8, the same set for the query.
    bf16x8 qv[KSTEPS];
    {
        const int m = rows_base + l32;
        const bool ok = m < a.M;
        const int r = ok ? m / a.G : 0, hh = ok ? m % a.G : 0;
        const uint16_t *qrow = (const uint16_t *)a.q +
                               (((int64_t)b * a.R + r) * a.Hq + (int64_t)g * a.G + hh) * D;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            const int ch = KVD ? 16 * (4 * (kk >> 2) + 2 * hl + ((kk >> 1) & 1)) + 8 * (kk & 1)
                               : 16 * kk + 8 * hl;
            int4 v4 = ok ? *(const int4 *)(qrow + ch) : make_int4(0, 0, 0, 0);
            qv[kk] = __builtin_bit_cast(bf16x8, v4);
        }
    }
#pragma unroll
    for (int j = 0; j < PTPT; ++j) {
        const int i = tid + j * THREADS;
        if (i < npt && i < kPtMax)
            pt[i] = (int32_t)clamp_page(ptv[j], a.num_pages);
    }
    __syncthreads();

    const int ps_mask = (1 << a.ps_shift) - 1;
    const uint32_t lds0 = lds_off(lds);
    // Loader roles, fixed for the whole kernel: load i of this thread fills
    // stage slot i*THREADS + tid, i.e. chunk (slot % CH) ^ swz(key) of key
    // slot / CH of the K region (first half of the slots) or the V region.
    const uint16_t *src_base[LPS];
    int ld_key[LPS];
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
        const int slot = i * THREADS + tid;
        const int region = (i * THREADS + w * 64) / (SK * CH);   // wave-uniform
        const int s2 = slot - region * (SK * CH);
        ld_key[i] = s2 / CH;
        src_base[i] = (const uint16_t *)(region ? a.v : a.k) + (int64_t)g * a.stride_head +
                      (((s2 % CH) ^ swz<D>(ld_key[i])) * 8);
    }

    // Issue the direct-to-LDS loads of stage st.  Load i of a wave covers KPI
    // consecutive keys (one per CH lanes); this lane's chunk position and
    // swizzle depend only on the key modulo 16, so its 32-bit offset is fixed.
    constexpr int KPI = 64 / CH;
    constexpr int LH = LPS / 2;   // loads per region (K, then V)
    // (with fewer threads than 16 keys' chunks, loads j of even and odd j
    // start at keys of either parity of 8, so a lane has two offsets)
    constexpr int NOFF = (THREADS / CH) % (D == 128 ? 16 : 8) == 0 ? 1 : 2;
    static_assert(NOFF == 1 || (2 * THREADS / CH) % (D == 128 ? 16 : 8) == 0, "swizzle period");
    uint32_t lane_off[NOFF];
#pragma unroll
    for (int jp = 0; jp < NOFF; ++jp)
        lane_off[jp] = (uint32_t)((lane / CH) * a.stride_token * 2 +
                                  (((lane % CH) ^ swz<D>((jp * THREADS + w * 64 + lane) / CH)) * 16));
    auto issue = [&](int st) {
        const uint32_t sbase = lds0 + (uint32_t)((st % NBUF) * SB);
        const int kst = kb0 + st * SK;
        if (wave_pages) {
            int32_t pgs[LH];
#pragma unroll
            for (int j = 0; j < LH; ++j) {
                const int k0 = kst + (j * THREADS + w * 64) / CH;
                pgs[j] = k0 < kr.hi ? pt[(k0 >> a.ps_shift) - lp0] : 0;
            }
#pragma unroll
            for (int i = 0; i < LPS; ++i) {
                const int j = i % LH;
                const int k0 = kst + (j * THREADS + w * 64) / CH;   // wave-uniform
                if (k0 >= kr.hi)
                    continue;
                const int t = k0 + lane / CH;
                const bool in = (k0 >= kr.lo && k0 + KPI <= kr.hi) || (t >= kr.lo && t < kr.hi);
                const int64_t off = (int64_t)__builtin_amdgcn_readfirstlane(pgs[j]) * a.stride_page +
                                    (int64_t)g * a.stride_head + (int64_t)(k0 & ps_mask) * a.stride_token;
                const uint16_t *base = (const uint16_t *)(i >= LH ? a.v : a.k) + off;
                if (in)
                    dma_load16_s(base, lane_off[j % NOFF], sbase + (i * THREADS + w * 64) * 16);
            }
        } else {
            int64_t page[LPS];
#pragma unroll
            for (int i = 0; i < LPS; ++i) {
                const int t = kst + ld_key[i];
                page[i] = t < kr.hi ? pt[(t >> a.ps_shift) - lp0] : 0;
            }
#pragma unroll
            for (int i = 0; i < LPS; ++i) {
                const int t = kst + ld_key[i];
                if (t < kr.hi)
                    dma_load16(src_base[i] + page[i] * a.stride_page +
                                   (int64_t)(t & ps_mask) * a.stride_token,
                               __builtin_amdgcn_readfirstlane(sbase + (i * THREADS + w * 64) * 16));
            }
        }
    };

    // The window keys P .. P + W - 1 (a fused launch) as rows 0 .. W - 1 of
    // one more stage, in buffer ns % NBUF, which no wave reads once the stage
    // loop is done (stage ns - NBUF, or no stage); page per lane.  It is
    // issued after the loop: inside it, its address arithmetic spilled the
    // loop's scalar registers.  Rows W ..
    // SK - 1 keep stale data: their scores are masked and their V values are
    // made finite before use.
    auto issue_window = [&]() {
        const uint32_t sbase = lds0 + (uint32_t)((ns % NBUF) * SB);
#pragma unroll
        for (int i = 0; i < LPS; ++i) {
            const int j = ld_key[i];
            if (j < a.W) {
                const int t = Pw + j;
                const int64_t page = pt[(t >> a.ps_shift) - lp0];
                dma_load16(src_base[i] + page * a.stride_page + (int64_t)(t & ps_mask) * a.stride_token,
                           __builtin_amdgcn_readfirstlane(sbase + (i * THREADS + w * 64) * 16));
            }
        }
    };

    // FP8 E4M3 rows of 128 channels: load i of wave w is load I = i WAVES + w
    // of the raw stage, region I / (SK / 8) (K, then V), keys 8 (I % (SK / 8))
    // .. +7 of the stage; lane l takes key + l / 8 and 16-byte position l % 8,
    // which holds chunk position ^ xk8(key) in a K row and position ^
    // yv8(key) in a V row.  Each load reads eight whole 128-byte rows.  The
    // swizzles depend on the key modulo 16 only, so a lane has one offset per
    // region and key-group parity.  xk8 puts the 32 keys of a K operand read
    // (one chunk) on every 16-byte bank slot twice; yv8 puts the 8 keys x 2
    // chunks (c and c + 4) of a 32-lane transposing V read on 16 distinct
    // slots.
    auto xk8s = [](int k) { return (k >> 1) & 7; };
    auto yv8s = [](int k) { return ((k >> 1) & 1) | ((k >> 2) & 2); };
    uint32_t loff8[2][2];
#pragma unroll
    for (int rg8 = 0; rg8 < 2; ++rg8)
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            const int key = 8 * par + (lane >> 3), pos = lane & 7;
            const int c = pos ^ (rg8 ? yv8s(key) : xk8s(key));
            loff8[rg8][par] = (uint32_t)((lane >> 3) * a.stride_token + c * 16);
        }
    auto issue8d = [&](int st) {
        const uint32_t sbase = lds0 + (uint32_t)((st % NBUF8) * SB8);
        const int kst = kb0 + st * SK;
        // the page of each load's key group, all read before the first load
        int32_t pg8[LPS8];
#pragma unroll
        for (int i = 0; i < LPS8; ++i) {
            const int k0 = kst + 8 * ((i * (THREADS / 64) + w) % (SK / 8));
            pg8[i] = wave_pages && k0 < kr.hi ? pt[(k0 >> a.ps_shift) - lp0] : 0;
        }
#pragma unroll
        for (int i = 0; i < LPS8; ++i) {
            const int I = i * (THREADS / 64) + w;                   // wave-uniform
            const int region = I / (SK / 8), kg8 = I % (SK / 8);
            const int k0 = kst + 8 * kg8;
            if (k0 >= kr.hi)
                continue;
            const int t = k0 + (lane >> 3);
            const bool in = (k0 >= kr.lo && k0 + 8 <= kr.hi) || (t >= kr.lo && t < kr.hi);
            const uint32_t dst = sbase + (uint32_t)(region * SK * D + kg8 * 1024);
            const uint8_t *src = (const uint8_t *)(region ? a.v : a.k) + (int64_t)g * a.stride_head;
            if (wave_pages) {
                const int64_t off = (int64_t)__builtin_amdgcn_readfirstlane(pg8[i]) * a.stride_page +
                                    (int64_t)(k0 & ps_mask) * a.stride_token;
                if (in)
                    dma_load16_s(src + off, loff8[region][kg8 & 1], dst);
            } else if (in) {
                const int key = 8 * kg8 + (lane >> 3);
                const int c = (lane & 7) ^ (region ? yv8s(key) : xk8s(key));
                dma_load16(src + (int64_t)pt[(t >> a.ps_shift) - lp0] * a.stride_page +
                               (int64_t)(t & ps_mask) * a.stride_token + c * 16,
                           dst);
            }
        }
    };

    // FP8 E4M3 rows of 64 channels: each thread loads its 16-byte chunks (16
    // values of one row) of a stage into registers and converts them into the
    // bf16 stage layout above, so the MFMA code is the bf16 code.  Two
    // register sets (stage x in set x & 1) keep two stages in flight.
    constexpr int C8 = D / 16;                                // 16-byte chunks per fp8 row
    constexpr int LP8 = (KV8 && !KVD) ? 2 * SK * C8 / THREADS : 1;   // chunks per thread and stage
    static_assert(!KV8 || KVD || (2 * SK * C8) % THREADS == 0, "fp8 slot split");
    int4 f8a[LP8], f8b[LP8];
    // Every load is issued, also for stages past the last one (keys at or
    // past the split end re-read its last key and are zeroed at conversion):
    // with no conditional loads the compiler's count of outstanding loads is
    // exact, and its wait for one set leaves the other in flight.
    auto load8 = [&](int st, int4 (&f8)[LP8]) {
        const int kst = kb0 + st * SK;
        int64_t page[LP8];
#pragma unroll
        for (int i = 0; i < LP8; ++i) {
            const int s2 = (i * THREADS + tid) % (SK * C8);
            const int t = min(kst + s2 / C8, kr.hi - 1);
            page[i] = pt[(t >> a.ps_shift) - lp0];
        }
#pragma unroll
        for (int i = 0; i < LP8; ++i) {
            const int slot = i * THREADS + tid;
            const int region = slot / (SK * C8), s2 = slot % (SK * C8);
            const int t = min(kst + s2 / C8, kr.hi - 1);
            const uint8_t *src = (const uint8_t *)(region ? a.v : a.k) + page[i] * a.stride_page +
                                 (int64_t)g * a.stride_head + (int64_t)(t & ps_mask) * a.stride_token +
                                 (s2 % C8) * 16;
            f8[i] = *(const int4 *)src;
        }
    };
    auto convert8 = [&](int st, const int4 (&f8)[LP8]) {
        char *buf = lds + (st % NBUF) * SB;
#pragma unroll
        for (int i = 0; i < LP8; ++i) {
            const int slot = i * THREADS + tid;
            const int region = slot / (SK * C8), s2 = slot % (SK * C8);
            const int key = s2 / C8, c8 = s2 % C8;
            int4 lo, hi;
            fp8x16_to_bf16(f8[i], lo, hi);
            if (kb0 + st * SK + key >= kr.hi)
                lo = hi = make_int4(0, 0, 0, 0);
            char *row = buf + region * (SB / 2) + key * ROWB;
            *(int4 *)(row + (((2 * c8) ^ swz<D>(key)) * 16)) = lo;
            *(int4 *)(row + (((2 * c8 + 1) ^ swz<D>(key)) * 16)) = hi;
        }
    };

    f32x16 o[DT];
    float m_run = -INFINITY, l_run = 0.f;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            o[t][r] = 0.f;

    // convert stage st + 1 (stage st + 2 stays in flight) and reuse its
    // register set for stage st + 3
    auto advance8 = [&](int st, int4 (&f8)[LP8]) {
        convert8(st + 1, f8);
        load8(st + 3, f8);
    };
    // Stage 0 goes out first, then the query is made ready (the compiler's
    // wait for it also covers the direct-to-LDS loads issued before, which
    // it does not count: only stage 0, which the first trip needs anyway),
    // then the rest of the prefetch.
    if constexpr (KVD) {
        if (ns > 0)
            issue8d(0);
    } else if constexpr (!KV8) {
        if (ns > 0)
            issue(0);
    }
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
        if constexpr (KV8)
            qv[kk] = bf16x8_round_e4m3(qv[kk]);
        settle(qv[kk]);
    }
    if constexpr (KVD) {
        for (int st = 1; st < NBUF8 - 1 && st < ns; ++st)
            issue8d(st);
    } else if constexpr (KV8) {
        if (ns > 0) {
            load8(0, f8a);
            load8(1, f8b);
            convert8(0, f8a);
            load8(2, f8a);
        }
    } else {
        for (int st = 1; st < NBUF - 1 && st < ns; ++st)
            issue(st);
    }

    const int G16 = lane >> 4, a4 = lane & 3, j4 = (lane >> 2) & 3;
    const int key0 = ks * 32;
    const int krow = key0 + l32;                 // K operand: key of this lane
    const int ksw = swz<D>(krow);
    // the row's ancestor mask over the window keys (a fused launch)
    uint64_t rmask = 0ull;
    // one stage of keys: S, softmax weights and O for this wave's 32 keys;
    // win: the window stage (keys P + key0 .. of buffer ns % NBUF), masked
    // per row, with the weights split into a bf16 head and remainder (a row
    // may weigh few window keys, whose rounding would not average out)
    // last: the last stage over bf16 K/V, whose rows past the split end are
    // not loaded (see the V operand below)
    auto compute = [&](int it, bool win, bool last) {
        const char *Kb = KVD ? lds + (it % NBUF8) * SB8 : lds + (it % NBUF) * SB;
        const char *Vb = KVD ? Kb + SK * D : Kb + SB / 2;
        const int first = kb0 + it * SK + key0;  // absolute key of this wave's block
        if (win ? key0 >= a.W : first >= kr.hi)
            return;
        // S^T[key][row] = sum_d K[key][d] Q[row][d]; FP8 rows: two E4M3 x
        // E4M3 steps of 64 channels (unit block scales), lane (key l32, half
        // hl) reading chunks 4 kk + 2 hl + e of its key row
        f32x16 s;
        if constexpr (KVD) {
            // E4M3 chunks widened exactly to bf16 in registers, bf16 MFMA
            const char *kr0 = Kb + krow * D;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[r] = 0.f;
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int4 x = *(const int4 *)(kr0 + (((4 * c + 2 * hl + e) ^ xk8s(krow)) * 16));
                    int4 lo, hi;
                    fp8x16_to_bf16(x, lo, hi);
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, lo),
                                                                qv[4 * c + 2 * e], s, 0, 0, 0);
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, hi),
                                                                qv[4 * c + 2 * e + 1], s, 0, 0, 0);
                }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[r] = 0.f;
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                const bf16x8 ka = *(const bf16x8 *)(Kb + krow * ROWB + (((2 * kk + hl) ^ ksw) * 16));
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qv[kk], s, 0, 0, 0);
            }
        }
        // keys outside the split are not visible; a window key only to the
        // rows whose mask has its bit
        if (win) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j = key0 + 8 * (r >> 2) + 4 * hl + (r & 3);
                if (!((rmask >> j) & 1ull))
                    s[r] = -INFINITY;
            }
        } else if (first < kr.lo || first + 32 > kr.hi) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = first + 8 * (r >> 2) + 4 * hl + (r & 3);
                if (key < kr.lo || key >= kr.hi)
                    s[r] = -INFINITY;
            }
        }
        // online softmax in the exp2 domain; the running max is only raised
        // when a block exceeds it by more than 2^8, so rescaling of O is rare
        // and weights stay <= 256
        float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
        for (int r = 3; r < 16; ++r)
            mx = fmaxf(mx, s[r]);
        mx = pair_max(mx);
        const float mb = mx * a.c;
        if (__ballot(mb > m_run + 8.f)) {
            const float mnew = fmaxf(m_run, mb);
            const float alpha = fast_exp2(m_run - mnew);  // 0 when m_run = -inf
            l_run *= alpha;
#pragma unroll
            for (int t = 0; t < DT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    o[t][r] *= alpha;
            m_run = mnew;
        }
        const float mu = m_run == -INFINITY ? 0.f : m_run;
        bf16x8 pb[2], prm[2];
        float lsum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pr = fast_exp2(fmaf(s[r], a.c, -mu));
            lsum += pr;
            const __bf16 ph = (__bf16)pr;
            pb[r >> 3][r & 7] = ph;
            if (win)
                prm[r >> 3][r & 7] = (__bf16)(pr - (float)ph);
        }
        l_run += lsum;
        // O^T[d][row] += sum_key V[key][d] P[row][key].  The P operand is the
        // S accumulator as is: the key order inside each 16-key chunk is
        // permuted identically for V (transposing LDS reads) and P, which
        // leaves the sum unchanged.  V^T operand of d tile t, chunk cc, half
        // hr: lane (G16, a4, j4) points at key key0 + 16 cc + 8 hr + 4 (G16/2)
        // + j4, channels d0 .. d0 + 3; the 16-lane group's read transposes
        // the 4 keys x 4 channels.
        if constexpr (KVD) {
            // FP8 rows: V^T operand of d tile t (channels 16 t .. +15 and
            // D / 2 + 16 t .. +15, as for bf16 rows), chunk cc, by one
            // transposing byte read per lane and a widening to bf16.  Lane j
            // of 16-lane group G16 points at key key0 + 16 cc + 4 hl + (e & 3)
            // + 8 (e >> 2), e = j / 2, bytes 8 (j & 1) .. +7 of chunk (G16 &
            // 1) D / 32 + t; the read hands lane i byte i % 8 of lanes 2 e + i
            // / 8, i.e. channel (G16 & 1) D / 2 + 16 t + i of the 8 keys, in
            // the key order of the P operand.
            typedef __attribute__((ext_vector_type(2))) int v2i;
            const int e8 = (lane & 15) >> 1;
            const int vkey = key0 + 4 * hl + (e8 & 3) + 8 * (e8 >> 2);
            const int vy = yv8s(vkey);
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                const int vc = ((G16 & 1) * (D / 32) + t) ^ vy;
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    const char *p = Vb + (vkey + 16 * cc) * D + vc * 16 + 8 * (lane & 1);
                    const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i *)p);
                    auto w0 = [](int x) {
                        return __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)x, 1.0f, false));
                    };
                    auto w1 = [](int x) {
                        return __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)x, 1.0f, true));
                    };
                    const int4 w4 = make_int4(w0(r.x), w1(r.x), w0(r.y), w1(r.y));
                    o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w4), pb[cc], o[t],
                                                                   0, 0, 0);
                }
            }
            return;
        }
        // A block of the last stage reaching past the split end has rows that
        // were not loaded; once the stage ring has come round they hold an
        // earlier stage's keys, whose weight here is exactly 0, and a +-inf V
        // value among them would turn into 0 * inf = NaN: those operand
        // elements are zeroed.  Element e of the V^T operand of chunk cc is
        // key 16 cc + 4 hl + 8 (e / 4) + e % 4 of the block.  (The last stage
        // runs outside the stage loop, so the loop carries none of this.)
        const int vlim = kr.hi - first - 4 * hl;
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            const int d0 = ((G16 & 1) ? D / 2 : 0) + 16 * t + 4 * a4;
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                i16x4 half[2];
#pragma unroll
                for (int hr = 0; hr < 2; ++hr) {
                    const int key = key0 + cc * 16 + hr * 8 + 4 * (G16 >> 1) + j4;
                    const char *p =
                        Vb + key * ROWB + (((d0 >> 3) ^ swz<D>(key)) * 16) + (a4 & 1) * 8;
                    half[hr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)p);
                }
                struct {
                    i16x4 lo, hi;
                } pair{half[0], half[1]};
                bf16x8 va = __builtin_bit_cast(bf16x8, pair);
                if (last && first + 32 > kr.hi) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (16 * cc + 8 * (e >> 2) + (e & 3) >= vlim)
                            va[e] = (__bf16)0.f;
                }
                o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[cc], o[t], 0, 0, 0);
                if (win)
                    o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, prm[cc], o[t], 0, 0, 0);
            }
        }
    };

    if constexpr (KVD) {
        for (int it = 0; it < ns; ++it) {
            // as for bf16 rows: stage `it` is complete once at most the loads
            // of the later, full stages are outstanding
            if (it + NBUF8 - 2 < ns - 1)
                wait_vmcnt<(NBUF8 - 2) * LPS8>();
            else
                wait_vmcnt<0>();
            __syncthreads();
            if (it + NBUF8 - 1 < ns)
                issue8d(it + NBUF8 - 1);
            compute(it, false, false);
        }
    } else if constexpr (KV8) {
        // Stage it was converted in the previous trip; after the barrier no
        // wave reads the buffer stage it + 1 is converted into.  Unrolled by
        // two so each trip names its register set statically; a trip past
        // the last stage computes nothing (its keys are all at or past the
        // split end).
        for (int it = 0; it < ns; it += 2) {
            __syncthreads();
            advance8(it, f8b);
            compute(it, false, false);
            __syncthreads();
            advance8(it + 1, f8a);
            compute(it + 1, false, false);
        }
    } else {
        for (int it = 0; it < ns - 1; ++it) {
            // Stage `it` is complete once at most the loads of the later, full
            // stages are outstanding.  When the last (partial) stage is among
            // the outstanding ones some of its instructions may be skipped, so
            // wait for everything then.
            if (it + NBUF - 2 < ns - 1)
                wait_vmcnt<(NBUF - 2) * LPS>();
            else
                wait_vmcnt<0>();
            __syncthreads();  // every wave's loads of stage it landed; stage it-1 is free
            if (it + NBUF - 1 < ns)
                issue(it + NBUF - 1);
            compute(it, false, false);
        }
        if (ns > 0) {
            // the last stage (nothing left to issue)
            wait_vmcnt<0>();
            __syncthreads();
            compute(ns - 1, false, true);
        }
    }

    // The window stage (a fused launch): once it has landed its non-finite V
    // values are set to 0 and their keys flagged, as in the window kernel;
    // then each wave takes its 32 window keys like a prefix block.  A row
    // that sees a flagged key gets those keys' non-finite values added to its
    // output below, which is what the exact weighted sum gives.
    if constexpr (FUSE) {
        if (wown) {
            issue_window();
            wait_vmcnt<0>();
            __syncthreads();
            char *vw = lds + (ns % NBUF) * SB + SB / 2;
            for (int i = tid; i < SB / 32; i += THREADS) {
                const int key = (i * 16) / ROWB;
                uint4 u4 = *(const uint4 *)(vw + i * 16);
                uint32_t x[4] = {u4.x, u4.y, u4.z, u4.w};
                bool nf = false;
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)
                        if (((x[e] >> (16 * h2)) & 0x7F80u) == 0x7F80u) {
                            nf = true;
                            x[e] &= ~(0xFFFFu << (16 * h2));
                        }
                if (nf) {
                    *(uint4 *)(vw + i * 16) = make_uint4(x[0], x[1], x[2], x[3]);
                    if (key < a.W)
                        atomicOr(&wbad[key >> 5], 1u << (key & 31));
                }
            }
            __syncthreads();
            rmask = wmk[l32];
            if (a.W < 64)
                rmask &= (1ull << a.W) - 1ull;
            compute(ns, true, false);
        }
    }

    // The split's partial (O / l, lse2) of each row.  The NKS key subsets of
    // a row block are combined here, as the merge combines partials: every
    // wave stores its normalised O (in its MFMA layout: lane and register
    // index name the same rows and channels in every wave) and its rows'
    // lse2 in the free stage buffers; then wave ks combines float4 units ks,
    // ks + NKS, ... of its row block and writes them.  The max is
    // NaN-propagating, so a NaN subset makes the row NaN.
    constexpr int NU = DT * 4;   // float4 units of a lane's O
    static_assert(C::WAVES * NU * 64 * 16 <= LDSB, "key-subset partials fit the stage buffers");
    __shared__ float cl[NRB * NKS][32];
    const float lt = pair_sum(l_run);
    const float inv = has_keys(lt) ? 1.f / lt : 0.f;
    __syncthreads();   // every wave is done with the stage buffers
    float4 *cb = reinterpret_cast<float4 *>(lds);
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            cb[(w * NU + 4 * t + q4) * 64 + lane] =
                make_float4(o[t][4 * q4] * inv, o[t][4 * q4 + 1] * inv, o[t][4 * q4 + 2] * inv,
                            o[t][4 * q4 + 3] * inv);
    if (hl == 0)
        cl[w][l32] = has_keys(lt) ? m_run + __log2f(lt) : -INFINITY;
    __syncthreads();
    float lk[NKS], z[NKS];
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < NKS; ++k) {
        lk[k] = cl[k * NRB + rbw][l32];
        mx = (lk[k] != lk[k] || mx != mx) ? __builtin_nanf("") : fmaxf(mx, lk[k]);
    }
    float zs = 0.f;
#pragma unroll
    for (int k = 0; k < NKS; ++k) {
        z[k] = lk[k] != -INFINITY ? fast_exp2(lk[k] - mx) : 0.f;
        zs += z[k];
    }
    const bool any = mx != -INFINITY;
    const float zinv = any ? 1.f / zs : 0.f;
    const int m = rows_base + l32;
    const bool fout = FUSE && a.fuse;   // the only split of a fused launch: write the output
    uint64_t vbad = rmask & (((uint64_t)wbad[1] << 32) | wbad[0]);
    if (m < a.M) {
        const int r = m / a.G, hh = m % a.G;
        const int64_t row = ((int64_t)b * a.R + r) * a.Hq + (int64_t)g * a.G + hh;
        float *dst = a.ws_o + (row * a.S + split) * D;
        for (int u = ks; u < NU; u += NKS) {
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int k = 0; k < NKS; ++k) {
                if (lk[k] != -INFINITY) {
                    const float4 v = cb[((k * NRB + rbw) * NU + u) * 64 + lane];
                    acc.x = fmaf(z[k], v.x, acc.x);
                    acc.y = fmaf(z[k], v.y, acc.y);
                    acc.z = fmaf(z[k], v.z, acc.z);
                    acc.w = fmaf(z[k], v.w, acc.w);
                }
            }
            const int t = u >> 2, q4 = u & 3;
            const int d = ((q4 >> 1) ? D / 2 : 0) + 16 * t + 8 * (q4 & 1) + 4 * hl;
            float res[4] = {acc.x * zinv, acc.y * zinv, acc.z * zinv, acc.w * zinv};
            if constexpr (FUSE) {
                // visible window keys with non-finite V values (rare): add those values
                for (uint64_t vb = vbad; vb; vb &= vb - 1) {
                    const int t_ = Pw + __ffsll((unsigned long long)vb) - 1;
                    const int64_t page =
                        clamp_page(a.page_table[(int64_t)b * a.max_pages + (t_ >> a.ps_shift)], a.num_pages);
                    const uint16_t *vr = (const uint16_t *)a.v + page * a.stride_page +
                                         (int64_t)g * a.stride_head + (int64_t)(t_ & ps_mask) * a.stride_token;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x = bf16_bits_to_f32(vr[d + e]);
                        if (!(fabsf(x) < INFINITY))
                            res[e] += x;
                    }
                }
            }
            if (fout) {
                const uint32_t lo = f32_to_bf16_bits(res[0]) | ((uint32_t)f32_to_bf16_bits(res[1]) << 16);
                const uint32_t hi = f32_to_bf16_bits(res[2]) | ((uint32_t)f32_to_bf16_bits(res[3]) << 16);
                *(uint2 *)((uint16_t *)a.out + row * D + d) = make_uint2(lo, hi);
            } else {
                *(float4 *)(dst + d) = make_float4(res[0], res[1], res[2], res[3]);
            }
        }
        const float lse = any ? mx + __log2f(zs) : -INFINITY;
        if (ks == 0 && hl == 0) {
            if (fout) {
                if (a.lse2)
                    a.lse2[row] = lse;
            } else {
                a.ws_lse[row * a.S + split] = lse;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Software-pipelined prefix kernel for wide row groups (256 folded rows:
// 8 waves x 32 rows, every wave reads every key).  Stages are 64 keys, NBUF
// deep, with one workgroup barrier per stage.  Per 32-key block u a wave
// issues the O^T += V^T P^T MFMAs of block u - 1 interleaved with the softmax
// weights of block u, then the S MFMAs of block u + 1, so the MFMA pipe
// works while the vector ALU computes exponentials (two waves per SIMD fill
// each other's gaps); each MFMA operand is read from LDS one phase ahead of
// its use.  The stage barrier would line both waves of a SIMD up on the same
// phase (both computing weights, then both waiting on their S chains), so
// waves 4..7, which share the SIMDs of waves 0..3 (waves are placed on the
// SIMDs round-robin), meet it before reading V and issuing the S chain
// instead of after: after each barrier one wave of a SIMD computes weights
// while the other runs its S MFMAs.  Either position is safe: a wave's reads
// of the stage being freed (the two blocks before the current one) are
// complete at both.
// The softmax reference max mu is taken from the first block and raised only
// when the running sum of weights would pass kSumLimit (rare): weights are
// bf16 with the fp32 exponent range and accumulate in fp32, so their
// magnitude costs no precision, and the common path needs no per-block row
// max.  A weight sum of at least 1 (the key that set mu) keeps every weight
// that underflows below 2^-126 negligible.
//
// LDS layout of a stage of SK keys.  The K and V regions are each a sequence of
// 128-byte pieces [chunk group cg][key k]: piece (cg, k) holds the 16-byte
// chunks 8 cg .. 8 cg + 7 of key k (one half row for D = 128), in the order
//   K: chunk 8 cg + (pos ^ xk(k)) at position pos, xk(k) = (k ^ ((k >> 3) & 1)) & 7
//   V: chunk 8 cg + (pos ^ yv(k, cg)) at position pos, yv = 2 ((k & 3) ^ (cg & 1))
// A direct-to-LDS load therefore always reads whole 128-byte lines (8 lanes per
// line, in permuted order, which still coalesces), and the operand reads are
// bank-conflict-free with 32 or 64 banks: the 8 (16) keys of one K read land
// on distinct 16-byte slots of a 128 (256) byte window, and the 4 keys x 32
// bytes of a transposing V read, with the neighbouring 16-lane group, on
// disjoint 32-byte slots.  Each lane reads through 4 precomputed K offsets
// (one per k step mod 4) and 4 V offsets (one per channel tile); chunk group,
// key chunk and block are immediates.
//
// Loads: every load instruction covers all SK keys of one chunk group, wave w
// taking keys 8 w .. 8 w + 7 of the stage.  With pages of 8 or more keys those
// 8 keys share one page, so the page base is wave-uniform (scalar registers)
// and a lane only adds a fixed 32-bit offset: stages then start at the 8-key
// boundary at or below the split start, and keys outside [lo, hi) are neither
// loaded nor visible.  Smaller pages take a per-lane page lookup.
__device__ inline int xk(int k) { return (k ^ ((k >> 3) & 1)) & 7; }
__device__ inline int yv(int k, int cg) { return 2 * ((k & 3) ^ (cg & 1)); }

constexpr float kSumLimit = 1048576.f;   // 2^20


template <int D, int SK_, bool KV8>
struct PipeCfg {
    static constexpr int WAVES = 8;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int SK = SK_;                // keys per stage
    static constexpr int BPS = SK / 32;           // 32-key blocks per stage
    static constexpr int KSTEPS = D / 16;
    static constexpr int DT = D / 32;
    static constexpr int KREG = SK * D * 2;       // bytes of the K region (bf16)
    static constexpr int SB = 2 * KREG;           // stage bytes (bf16)
    // FP8 E4M3 caches: a ring of F8 raw stages (K then V, half the bytes of
    // a bf16 stage) and a ring of NBUF stages of V widened to bf16 (KREG
    // bytes each).  The scores read the raw K directly.
    static constexpr int F8 = 6;
    static constexpr int SB8 = SB / 2;
    static constexpr int LPS8 = SB8 / (THREADS * 16);
    static constexpr int NBUF0 = kLdsStageBudget / SB;
    static constexpr int NBUF = KV8 ? 3 : (NBUF0 > 12 ? 12 : NBUF0);
    static_assert(!KV8 || (LPS8 == 2 && SB8 % (THREADS * 16) == 0 && NBUF * KREG + F8 * SB8 <= kLdsStageBudget),
                  "fp8 stage split");
    static_assert(!KV8 || D == 128, "fp8 scores take two 64-channel MFMA steps");
    static constexpr int PF = NBUF - 2;           // stages in flight ahead of the current one
    static constexpr int LPS = SB / (THREADS * 16);
    static_assert(THREADS == SK * 8, "one load instruction covers every key of a stage");
    static_assert(BPS == 2, "block u + 2 starts a stage exactly when u is even");
    static_assert(NBUF >= 3 && LPS >= 1 && SB % (THREADS * 16) == 0, "stage split");
    static_assert((PF - 1) * LPS < 64, "vmcnt range");
};

template <int D, int SK_, bool KV8>
__global__ void __launch_bounds__(512, 1) k_prefix_mfma_pipe(PrefixArgs a) {
    using C = PipeCfg<D, SK_, KV8>;
    constexpr int BPS = C::BPS;
    constexpr int SK = C::SK, SB = C::SB, NBUF = C::NBUF, PF = C::PF, LPS = C::LPS,
                  THREADS = C::THREADS, KREG = C::KREG, KSTEPS = C::KSTEPS, DT = C::DT;
    constexpr int ROWS_WG = 256;

    constexpr int F8 = C::F8, SB8 = C::SB8, LPS8 = C::LPS8;
    // bf16: NBUF stages of K and V; FP8: NBUF stages of widened V, then the
    // F8 raw stages
    constexpr int VRING = KV8 ? NBUF * KREG : NBUF * SB;
    __shared__ __attribute__((aligned(16))) char lds[VRING + (KV8 ? F8 * SB8 : 0)];
    __shared__ int32_t pt[kPtMax];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane >> 5;
    const int l32 = lane & 31;

    const int units = a.B * a.Hkv * a.n_split;
    int rg, unit;
    const int id = blockIdx.x;
    if (a.RG > 1 && (units & 7) == 0) {
        const int xcd = id & 7, slot = id >> 3;
        rg = slot % a.RG;
        unit = (slot / a.RG) * 8 + xcd;
    } else {
        rg = id % a.RG;
        unit = id / a.RG;
    }
    const int split = unit % a.n_split;
    const int g = (unit / a.n_split) % a.Hkv;
    const int b = unit / (a.n_split * a.Hkv);

    const KeyRange kr = split_range(a, b, split);
    const bool wave_pages = !KV8 && a.ps_shift >= 3;
    // stages cover [kb0, hi); kb0 is in the page of lo
    const int kb0 = wave_pages ? (kr.lo & ~7) : kr.lo;
    const int nkeys = kr.hi > kr.lo ? kr.hi - kb0 : 0;
    const int ns = (nkeys + SK - 1) / SK;
    const int nb = (nkeys + 31) / 32;
    const int rows_base = rg * ROWS_WG + w * 32;

    // A fused launch (one split, whose range ends at the prefix length P):
    // the page-table slice also covers the window keys P .. P + W - 1.
    int Pw = 0;
    const bool wown = !KV8 && a.fuse && a.W > 0;
    if (wown) {
        Pw = a.prefix_len[b];
        Pw = Pw < 0 ? 0 : (Pw > a.max_prefix_len ? a.max_prefix_len : Pw);
    }
    const bool any_pt = nkeys > 0 || wown;
    const int lp0 = any_pt ? ((nkeys > 0 ? kb0 : Pw) >> a.ps_shift) : 0;
    const int npt = any_pt ? (((wown ? Pw + a.W : kr.hi) - 1) >> a.ps_shift) - lp0 + 1 : 0;
    for (int i = tid; i < npt && i < kPtMax; i += THREADS)
        pt[i] = (int32_t)clamp_page(a.page_table[(int64_t)b * a.max_pages + lp0 + i], a.num_pages);
    for (int i = tid; i < VRING / 16; i += THREADS)
        reinterpret_cast<int4 *>(lds)[i] = make_int4(0, 0, 0, 0);
    __shared__ uint32_t wbad[2];   // window keys 0..31, 32..63 with a non-finite V value
    if (tid < 2)
        wbad[tid] = 0u;
    // the window owner's row masks, fetched with the page table
    __shared__ uint64_t wmk[KV8 ? 1 : ROWS_WG];
    if (wown && tid < ROWS_WG) {
        const int mm = rg * ROWS_WG + tid;
        wmk[tid] = mm < a.M ? a.masks[(int64_t)b * a.R + mm / a.G] : 0ull;
    }

    // Q^T operand, bf16: lane (row l32, half hl) holds 8 channels of Q[row]
    // per 16-channel k step, 16 kk + 8 hl .. +8.  Under an FP8 cache the
    // query is rounded to E4M3 (held as bf16) and the E4M3 keys are widened
    // to bf16 in registers, so the products are exact and accumulate in fp32
    // (the FP8 MFMAs sum each 64-product group at about 12 bits relative to
    // its largest product).  The K operand lane then reads whole 16-byte
    // E4M3 chunks 4 c + 2 hl + e (c, e = 0, 1), and step 4 c + 2 e + h takes
    // channels 16 (4 c + 2 hl + e) + 8 h .. +8, for the query as well.
    bf16x8 qv[KSTEPS];
    {
        const int m = rows_base + l32;
        const bool ok = m < a.M;
        const int r = ok ? m / a.G : 0, hh = ok ? m % a.G : 0;
        const uint16_t *qrow = (const uint16_t *)a.q +
                               (((int64_t)b * a.R + r) * a.Hq + (int64_t)g * a.G + hh) * D;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            const int ch = KV8 ? 16 * (4 * (kk >> 2) + 2 * hl + ((kk >> 1) & 1)) + 8 * (kk & 1)
                               : 16 * kk + 8 * hl;
            int4 v4 = ok ? *(const int4 *)(qrow + ch) : make_int4(0, 0, 0, 0);
            qv[kk] = __builtin_bit_cast(bf16x8, v4);
            if constexpr (KV8)
                qv[kk] = bf16x8_round_e4m3(qv[kk]);
        }
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            settle(qv[kk]);
    }
    __syncthreads();

    // Loader roles (fixed): load i of a stage fills LDS slot i * THREADS + tid,
    // i.e. chunk group cg(i), key 8 w + (lane >> 3), position lane & 7.
    const int ps_mask = (1 << a.ps_shift) - 1;
    const uint32_t lds0 = lds_off(lds);
    const int key_l = lane >> 3;
    const int wkey = 8 * w + key_l;
    // element offset of this lane's 16-byte chunk within its key's row, per load
    auto chunk = [&](int i) {
        const bool vreg = i * THREADS >= SK * (D / 8);
        const int cg = (vreg ? i * THREADS - SK * (D / 8) : i * THREADS) / (SK * 8);
        return cg * 8 * 8 + ((lane & 7) ^ (vreg ? yv(wkey, cg) : xk(wkey))) * 8;
    };
    uint32_t ld_off[LPS];   // byte offsets of this lane's chunks from its key's row
#pragma unroll
    for (int i = 0; i < LPS; ++i)
        ld_off[i] = (uint32_t)(chunk(i) * 2);
    const uint32_t lane_tok = (uint32_t)(key_l * a.stride_token * 2);
    auto issue = [&](int st) {
        const uint32_t sbase = lds0 + (uint32_t)((st % NBUF) * SB) + w * 64 * 16;
        const int k0 = kb0 + st * SK + 8 * w;   // this wave's first key (wave-uniform)
        if (k0 >= kr.hi)
            return;
        const int t = k0 + key_l;
        const bool in = (k0 >= kr.lo && k0 + 8 <= kr.hi) || (t >= kr.lo && t < kr.hi);
        if (wave_pages) {
            const int64_t pg = __builtin_amdgcn_readfirstlane(pt[(k0 >> a.ps_shift) - lp0]);
            const int64_t off = pg * a.stride_page + (int64_t)g * a.stride_head +
                                (int64_t)(k0 & ps_mask) * a.stride_token;
            const uint16_t *kp = (const uint16_t *)a.k + off;
            const uint16_t *vp = (const uint16_t *)a.v + off;
            if (in) {
#pragma unroll
                for (int i = 0; i < LPS; ++i) {
                    const bool vreg = i * THREADS >= SK * (D / 8);
                    dma_load16_s(vreg ? vp : kp, lane_tok + ld_off[i], sbase + i * THREADS * 16);
                }
            }
        } else {
            const int64_t page = in ? pt[(t >> a.ps_shift) - lp0] : 0;
            const int64_t off = page * a.stride_page + (int64_t)g * a.stride_head +
                                (int64_t)(t & ps_mask) * a.stride_token;
            if (in) {
#pragma unroll
                for (int i = 0; i < LPS; ++i) {
                    const bool vreg = i * THREADS >= SK * (D / 8);
                    dma_load16((const uint16_t *)(vreg ? a.v : a.k) + off + chunk(i),
                               sbase + i * THREADS * 16);
                }
            }
        }
    };
    // The window keys P .. P + W - 1 as rows 0 .. W - 1 of one more stage, in
    // buffer ns % NBUF, which no prefix stage uses once stage ns - PF is
    // ready: it goes out with the prefix stages when they all fit in the
    // first PF slots, else after the main loop, before the last blocks
    // (outside the loop, so that it adds nothing to the loop's registers).  Page per
    // lane (the window need not start on an 8-key boundary).  Rows W .. 63
    // keep stale stage data: their scores are masked and their V values are
    // made finite before use.
    auto issue_window = [&]() {
        if (8 * w >= a.W)
            return;
        // (from an opaque copy of the lane index, so that nothing of this
        // once-per-workgroup path is shared with, or hoisted into, the loop)
        int l = lane;
        settle(l);
        const int j = 8 * w + (l >> 3);
        if (j < a.W) {
            const uint32_t sbase = lds0 + (uint32_t)((ns % NBUF) * SB) + w * 64 * 16;
            const int t = Pw + j;
            const int64_t off = (int64_t)pt[(t >> a.ps_shift) - lp0] * a.stride_page +
                                (int64_t)g * a.stride_head + (int64_t)(t & ps_mask) * a.stride_token;
#pragma unroll
            for (int i = 0; i < LPS; ++i) {
                const bool vreg = i * THREADS >= SK * (D / 8);
                const int cg = (vreg ? i * THREADS - SK * (D / 8) : i * THREADS) / (SK * 8);
                const int c = cg * 8 * 8 + ((l & 7) ^ (vreg ? yv(j, cg) : xk(j))) * 8;
                dma_load16((const uint16_t *)(vreg ? a.v : a.k) + off + c, sbase + i * THREADS * 16);
            }
        }
    };
    // Stage st is complete once at most the loads of the later, full stages
    // are outstanding (all of them when the partial last stage is among
    // them); then the barrier publishes every wave's loads and frees the
    // buffer of stage st - 2 for stage st + PF.
    auto stage_ready_bf16 = [&](int st) {
        if (st + PF - 1 < ns - 1)
            wait_vmcnt<(PF - 1) * LPS>();
        else
            wait_vmcnt<0>();
        __syncthreads();
        if (st + PF < ns)
            issue(st + PF);
    };

    // FP8 E4M3 caches.  A raw stage is SK key rows of D bytes of K, then of
    // V; thread tid loads 16-byte slot tid of each: key tid / 8, position
    // tid % 8.  K rows are read by every wave as the MFMA operand, with
    // position p of key k holding chunk p ^ xk8(k) (conflict-free operand
    // reads: the 16 keys of a 16-lane group land on distinct 16-byte slots
    // of 256 bytes).  The thread that loads a V chunk widens it (after its
    // own load has landed) into bf16 chunks 2 c8 and 2 c8 + 1 of the piece
    // layout, so V needs no barrier between the raw and the widened ring.
    // At stage_ready8(st) the raw stages issued are those up to st + F8 - 3;
    // stage st + 1 must have landed (its V is widened now, its K is read
    // after the next barrier) and the buffer of stage st - 2, which no wave
    // reads any more, takes stage st + F8 - 2.
    static_assert(!KV8 || D / 16 == 8, "one raw row is 8 chunks");
    auto xk8 = [](int k) { return (k >> 1) & 7; };
    const uint32_t lds8 = lds0 + (uint32_t)VRING;
    const int key8 = tid >> 3, pos8 = tid & 7;
    auto issue8 = [&](int st) {
        const int t = kb0 + st * SK + key8;
        const uint32_t rbase = lds8 + (uint32_t)((st % F8) * SB8) + w * 64 * 16;
        if (t < kr.hi) {
            const int64_t off = (int64_t)pt[(t >> a.ps_shift) - lp0] * a.stride_page +
                                (int64_t)g * a.stride_head + (int64_t)(t & ps_mask) * a.stride_token;
            dma_load16((const uint8_t *)a.k + off + ((pos8 ^ xk8(key8)) * 16), rbase);
            dma_load16((const uint8_t *)a.v + off + pos8 * 16, rbase + THREADS * 16);
        }
    };
    auto convert8 = [&](int st) {
        const char *raw = lds + VRING + (st % F8) * SB8 + SB8 / 2 + tid * 16;
        char *buf = lds + (st % NBUF) * KREG;
        int4 x = make_int4(0, 0, 0, 0);
        if (kb0 + st * SK + key8 < kr.hi)
            x = *(const int4 *)raw;
        int4 h[2];
        fp8x16_to_bf16(x, h[0], h[1]);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int c = 2 * pos8 + e, cg = c / 8;
            const int pos = (c % 8) ^ yv(key8, cg);
            *(int4 *)(buf + cg * (SK * 128) + key8 * 128 + pos * 16) = h[e];
        }
    };
    auto stage_ready8 = [&](int st) {
        if (st + 1 < ns) {
            if (st + F8 - 3 <= ns - 2)
                wait_vmcnt<(F8 - 4) * LPS8>();
            else
                wait_vmcnt<0>();
        }
        __syncthreads();
        if (st + 1 < ns)
            convert8(st + 1);
        if (st + F8 - 2 < ns)
            issue8(st + F8 - 2);
    };
    auto stage_ready = [&](int st) {
        if constexpr (KV8)
            stage_ready8(st);
        else
            stage_ready_bf16(st);
    };

    // per-lane operand offsets inside a stage (piece layout)
    constexpr int CGB = SK * 128;            // bytes per chunk group
    uint32_t koff[4], voff[DT];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        koff[q] = l32 * 128 + (((2 * q + hl) ^ xk(l32)) * 16);
    const int G16 = lane >> 4, a4 = lane & 3, j4 = (lane >> 2) & 3;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
        const int c = (G16 & 1) * (D / 16) + 2 * t + (a4 >> 1);   // chunk of channels d0..d0+3
        const int cg = c / 8, key = 4 * (G16 >> 1) + j4;
        voff[t] = cg * CGB + key * 128 + (((c % 8) ^ yv(key, cg)) * 16) + (a4 & 1) * 8;
    }

    f32x16 o[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            o[t][r] = 0.f;
    float mu = 0.f;      // reference max of the weights (exp2 domain, finite)
    float l_run = 0.f;

    auto block_base = [&](int u) { return lds + ((u / BPS) % NBUF) * SB + (u % BPS) * (32 * 128); };
    // V region of block u (the widened ring for FP8)
    auto vblock_base = [&](int u) {
        if constexpr (KV8)
            return lds + ((u / BPS) % NBUF) * KREG + (u % BPS) * (32 * 128);
        else
            return block_base(u) + KREG;
    };
    // FP8 K operand: lane (key l32, half hl) reads E4M3 chunks 4 c + 2 hl + e
    // (channels 16 (4 c + 2 hl + e) .. +16) of its key row, c, e = 0, 1
    uint32_t koff8[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int e = 0; e < 2; ++e)
            koff8[kk][e] = l32 * D + (((4 * kk + 2 * hl + e) ^ xk8(l32)) * 16);
    auto load_k = [&](int u, bf16x8 (&ka)[KSTEPS]) {
        if constexpr (KV8) {
            // E4M3 chunk 4 c + 2 hl + e -> bf16 steps 4 c + 2 e, 4 c + 2 e + 1
            const char *kb = lds + VRING + ((u / BPS) % F8) * SB8 + (u % BPS) * (32 * D);
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    int4 lo, hi;
                    fp8x16_to_bf16(*(const int4 *)(kb + koff8[c][e]), lo, hi);
                    ka[4 * c + 2 * e] = __builtin_bit_cast(bf16x8, lo);
                    ka[4 * c + 2 * e + 1] = __builtin_bit_cast(bf16x8, hi);
                }
        } else {
            const char *kb = block_base(u);
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk)
                ka[kk] = *(const bf16x8 *)(kb + (kk / 4) * CGB + koff[kk % 4]);
        }
    };
    auto load_v = [&](int u, bf16x8 (&va)[DT][2]) {
        const char *vb = vblock_base(u);
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const char *p = vb + voff[t] + cc * (16 * 128);
                struct {
                    i16x4 lo, hi;
                } pair{__builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)p),
                       __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(p + 8 * 128))};
                va[t][cc] = __builtin_bit_cast(bf16x8, pair);
            }
    };
    // S^T of one block: keys x rows, lane l holding row l % 32.
    auto qk = [&](const auto &ka) {
        f32x16 acc;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], qv[kk], kk ? acc : f32x16{}, 0, 0, 0);
        return acc;
    };
    // bf16 weights of one block and their sum (the values the MFMA multiplies)
    auto weights = [&](const f32x16 &sv, bf16x8 (&pb)[2], float &lb) {
        // the sum is taken over the fp32 weights: with few dominant keys the
        // bf16 rounding of the MFMA operand would not average out of lse2
        float l0 = 0.f, l1 = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(fmaf(sv[r], a.c, -mu));
            pb[r >> 3][r & 7] = (__bf16)p;
            if (r & 1)
                l1 += p;
            else
                l0 += p;
        }
        lb = l0 + l1;
    };
    auto row_max = [&](const f32x16 &sv) {
        float mx = fmaxf(fmaxf(sv[0], sv[1]), sv[2]);
#pragma unroll
        for (int r = 3; r < 16; ++r)
            mx = fmaxf(mx, sv[r]);
        return pair_max(mx) * a.c;
    };
    // Raise the reference to this block's row max, rescale what has been
    // accumulated, and recompute the block's weights.
    auto rebase = [&](const f32x16 &sv, bf16x8 (&pb)[2], float &lb) {
        const float mx = row_max(sv);
        const float mnew = mx < INFINITY ? fmaxf(mu, mx) : mu;
        const float alpha = fast_exp2(mu - mnew);
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                o[t][r] *= alpha;
        mu = mnew;
        weights(sv, pb, lb);
    };
    // rebase when the running sum would pass kSumLimit, then count the block
    auto check = [&](const f32x16 &sv, bf16x8 (&pb)[2], float lb) {
        if (__ballot(!(l_run + lb <= kSumLimit)))
            rebase(sv, pb, lb);
        l_run += lb;
    };
    // O^T += V^T P^T for one block
    auto pv = [&](const bf16x8 (&va)[DT][2], const bf16x8 (&pb)[2]) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int t = 0; t < DT; ++t)
                o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t][cc], pb[cc], o[t], 0, 0, 0);
    };
    // scores of keys outside [lo, hi) of the split become -inf (block u)
    auto mask_block = [&](f32x16 &sv, int u) {
        const int k0 = kb0 + u * 32 + 4 * hl;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + 8 * (r >> 2) + (r & 3);
            if (key < kr.lo || key >= kr.hi)
                sv[r] = -INFINITY;
        }
    };

    // One block u (1 <= u <= nb - 2).  Phase 1: O accumulates block u - 1 on
    // the MFMA pipe while the vector ALU turns S of block u into weights.
    // Phase 2: the V operands of block u are read, S of block u + 1 runs on
    // the MFMA pipe (into the registers S of block u has left), and the K
    // operands of block u + 2 are read.  Each LDS read lands during the
    // other phase; the two waves of a SIMD fill each other's gaps.  Every
    // block but the last is full.
    auto step = [&](int u, f32x16 &s, const bf16x8 (&pb_prev)[2], bf16x8 (&pb_cur)[2],
                    bool new_stage, auto &ka, bf16x8 (&va)[DT][2]) {
        float lb;
        pv(va, pb_prev);
        weights(s, pb_cur, lb);
#pragma unroll
        for (int i = 0; i < 2 * DT; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // O MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);    // weights VALU
        }
        check(s, pb_cur, lb);
        // waves 4..7 meet the stage barrier half a block before waves 0..3
        const bool early = !KV8 && w >= 4;
        if (early && new_stage && u + 2 < nb)
            stage_ready((u + 2) / BPS);
        load_v(u, va);
        s = qk(ka);
        if (u + 2 < nb) {
            if (new_stage && !early)
                stage_ready((u + 2) / BPS);
            load_k(u + 2, ka);
        }
    };

    if constexpr (KV8) {
        // raw stages 0 .. F8 - 3 in flight; widen V of stage 0 once its own
        // loads have landed
        for (int st = 0; st < F8 - 2 && st < ns; ++st)
            issue8(st);
        if (ns > 0) {
            if (F8 - 3 <= ns - 2)
                wait_vmcnt<(F8 - 3) * LPS8>();
            else
                wait_vmcnt<0>();
            convert8(0);
        }
    } else {
        for (int st = 0; st < PF && st < ns; ++st)
            issue(st);
        if (wown && ns < PF)
            issue_window();
    }
    if (nb > 0) {
        stage_ready(0);
        bf16x8 ka[KSTEPS];
        bf16x8 va[DT][2], pa[2], pbb[2];
        f32x16 s;
        load_k(0, ka);
        s = qk(ka);
        __builtin_amdgcn_sched_barrier(0);
        if (nb > 1)
            load_k(1, ka);   // block 1 is in stage 0
        mask_block(s, 0);
        mu = row_max(s);
        mu = fabsf(mu) < INFINITY ? mu : 0.f;
        if (nb == 1) {
            float lb;
            load_v(0, va);
            weights(s, pa, lb);
            check(s, pa, lb);
            pv(va, pa);
        } else {
            {
                // block 0 (no O work yet)
                float lb;
                weights(s, pa, lb);
                check(s, pa, lb);
                load_v(0, va);
                s = qk(ka);
                if (nb > 2) {
                    stage_ready(1);
                    load_k(2, ka);
                }
            }
            // blocks 1 .. nb - 2, two per trip so that the weight registers
            // alternate roles without copies; block u + 2 starts a stage
            // exactly when u is even
            int u = 1;
            for (; u + 1 <= nb - 2; u += 2) {
                step(u, s, pa, pbb, false, ka, va);
                step(u + 1, s, pbb, pa, true, ka, va);
            }
            if (wown && ns >= PF)
                issue_window();
            if (u == nb - 2) {
                step(u, s, pa, pbb, false, ka, va);
                pa[0] = pbb[0];
                pa[1] = pbb[1];
            }
            // the last block may be partial: keys past the split are not visible
            float lb;
            pv(va, pa);
            mask_block(s, nb - 1);
            weights(s, pbb, lb);
            check(s, pbb, lb);
            load_v(nb - 1, va);
            // Its rows past the split end are not loaded; once the stage ring
            // has come round they hold an earlier stage's keys, whose weight
            // here is exactly 0, and a +-inf V value among them would turn
            // into 0 * inf = NaN.  Element e of a V^T operand is key 16 cc +
            // 4 hl + 8 (e / 4) + e % 4 of the block (the P operand's order).
            {
                const int lim = kr.hi - (kb0 + (nb - 1) * 32 + 4 * hl);
#pragma unroll
                for (int t = 0; t < DT; ++t)
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (16 * cc + 8 * (e >> 2) + (e & 3) >= lim)
                                va[t][cc][e] = (__bf16)0.f;
            }
            pv(va, pbb);
        }
    }

    // The window part (a fused launch): once the window stage has
    // landed, its non-finite V values are set to 0 and their keys flagged;
    // then its (at most two) 32-key blocks run as prefix blocks do, with each
    // row's ancestor mask on the scores and the weights split into a bf16
    // head and remainder (a row may weigh few window keys, whose rounding
    // would not average out).  A row that sees a flagged key gets, per
    // channel, the sum of those keys' non-finite values added to its output,
    // which is what the exact weighted sum gives.
    const int m = rows_base + l32;
    uint64_t rmask = 0ull;
    if (wown) {
        wait_vmcnt<0>();
        __syncthreads();
        char *vw = lds + (ns % NBUF) * SB + KREG;
        for (int i = tid; i < KREG / 16; i += THREADS) {
            const int key = (i % (SK * 8)) / 8;
            uint4 u4 = *(const uint4 *)(vw + i * 16);
            uint32_t x[4] = {u4.x, u4.y, u4.z, u4.w};
            bool nf = false;
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
                    if (((x[e] >> (16 * h2)) & 0x7F80u) == 0x7F80u) {
                        nf = true;
                        x[e] &= ~(0xFFFFu << (16 * h2));
                    }
            if (nf) {
                *(uint4 *)(vw + i * 16) = make_uint4(x[0], x[1], x[2], x[3]);
                if (key < a.W)
                    atomicOr(&wbad[key >> 5], 1u << (key & 31));
            }
        }
        __syncthreads();
        rmask = wmk[w * 32 + l32];
        if (a.W < 64)
            rmask &= (1ull << a.W) - 1ull;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb * 32 >= a.W)
                break;
            const int u = ns * BPS + kb;   // the window stage's blocks
            bf16x8 ka[KSTEPS];
            load_k(u, ka);
            f32x16 sv = qk(ka);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int j = kb * 32 + 8 * (e >> 2) + 4 * hl + (e & 3);
                if (!((rmask >> j) & 1ull))
                    sv[e] = -INFINITY;
            }
            if (nb == 0 && kb == 0) {
                // no prefix keys: the reference is this block's row max
                mu = row_max(sv);
                mu = fabsf(mu) < INFINITY ? mu : 0.f;
            }
            bf16x8 pb[2], pr[2];
            float lb;
            auto wweights = [&]() {
                float l0 = 0.f, l1 = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(fmaf(sv[r], a.c, -mu));
                    const __bf16 ph = (__bf16)p;
                    pb[r >> 3][r & 7] = ph;
                    pr[r >> 3][r & 7] = (__bf16)(p - (float)ph);
                    if (r & 1)
                        l1 += p;
                    else
                        l0 += p;
                }
                lb = l0 + l1;
            };
            wweights();
            if (__ballot(!(l_run + lb <= kSumLimit))) {
                const float mx = row_max(sv);
                const float mnew = mx < INFINITY ? fmaxf(mu, mx) : mu;
                const float alpha = fast_exp2(mu - mnew);
                l_run *= alpha;
#pragma unroll
                for (int t = 0; t < DT; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        o[t][r] *= alpha;
                mu = mnew;
                wweights();
            }
            l_run += lb;
            bf16x8 va[DT][2];
            load_v(u, va);
            pv(va, pb);
            pv(va, pr);
        }
    }

    const int sidx = split;
    const float lt = pair_sum(l_run);
    if (m < a.M) {
        const int r = m / a.G, hh = m % a.G;
        const int64_t row = ((int64_t)b * a.R + r) * a.Hq + (int64_t)g * a.G + hh;
        const float inv = has_keys(lt) ? 1.f / lt : 0.f;
        // (an infinite weight sum comes only from a +inf score, whose exact
        // softmax, and so lse2, is NaN)
        const float lse = !has_keys(lt) ? -INFINITY : (lt < INFINITY ? mu + __log2f(lt) : __builtin_nanf(""));
        // lane value o[t][e] is channel chan(t, e) of row m
        auto chan = [&](int t, int e) {
            return ((e >> 3) ? D / 2 : 0) + 16 * t + 8 * ((e >> 2) & 1) + 4 * hl + (e & 3);
        };
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                o[t][e] *= inv;
        uint64_t vbad = rmask & (((uint64_t)wbad[1] << 32) | wbad[0]);
        if (wown && __ballot(vbad != 0ull)) {
            while (vbad) {
                const int j = __ffsll((unsigned long long)vbad) - 1;
                vbad &= vbad - 1;
                const int t_ = Pw + j;
                const int64_t page =
                    clamp_page(a.page_table[(int64_t)b * a.max_pages + (t_ >> a.ps_shift)], a.num_pages);
                const int64_t vo = page * a.stride_page + (int64_t)g * a.stride_head +
                                   (int64_t)(t_ & ps_mask) * a.stride_token;
#pragma unroll
                for (int t = 0; t < DT; ++t)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const float x = bf16_bits_to_f32(((const uint16_t *)a.v)[vo + chan(t, e)]);
                        if (!(fabsf(x) < INFINITY))
                            o[t][e] += x;
                    }
            }
        }
        if (!KV8 && a.fuse) {
            // a fused launch: this is the row's output
            uint16_t *out = (uint16_t *)a.out + row * D;
#pragma unroll
            for (int t = 0; t < DT; ++t)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const uint32_t lo = f32_to_bf16_bits(o[t][4 * q4]) |
                                        ((uint32_t)f32_to_bf16_bits(o[t][4 * q4 + 1]) << 16);
                    const uint32_t hi = f32_to_bf16_bits(o[t][4 * q4 + 2]) |
                                        ((uint32_t)f32_to_bf16_bits(o[t][4 * q4 + 3]) << 16);
                    *(uint2 *)(out + chan(t, 4 * q4)) = make_uint2(lo, hi);
                }
            if (a.lse2 && hl == 0)
                a.lse2[row] = lse;
        } else {
            float *dst = a.ws_o + (row * a.S + sidx) * D;
#pragma unroll
            for (int t = 0; t < DT; ++t)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    *(float4 *)(dst + chan(t, 4 * q4)) = make_float4(o[t][4 * q4], o[t][4 * q4 + 1],
                                                                     o[t][4 * q4 + 2], o[t][4 * q4 + 3]);
            if (hl == 0)
                a.ws_lse[row * a.S + sidx] = lse;
        }
    }
}

// fp32 prefix: one wave per (row, split); lanes over keys for the scores,
// lanes over channels for the weighted sum of values.
template <int D>
__global__ void __launch_bounds__(64) k_prefix_f32(PrefixArgs a) {
    constexpr int VPL = D / 64;
    __shared__ float qs[D];
    __shared__ float pw[64];
    __shared__ int64_t offs[64];
    const int lane = threadIdx.x;
    const int64_t gw = blockIdx.x;
    const int64_t row = gw / a.n_split;
    const int split = (int)(gw % a.n_split);
    const int h = (int)(row % a.Hq);
    const int b = (int)(row / ((int64_t)a.Hq * a.R));
    const int g = h / a.G;
    const float *q = (const float *)a.q + row * D;
    const float *kp = (const float *)a.k + (int64_t)g * a.stride_head;
    const float *vp = (const float *)a.v + (int64_t)g * a.stride_head;
    for (int d = lane; d < D; d += 64)
        qs[d] = q[d];
    __syncthreads();
    const KeyRange kr = split_range(a, b, split);
    const int ps_mask = (1 << a.ps_shift) - 1;
    float m = -INFINITY, l = 0.f, o[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        o[i] = 0.f;
    for (int base = kr.lo; base < kr.hi; base += 64) {
        const int t = base + lane;
        const bool valid = t < kr.hi;
        float u = -INFINITY;
        int64_t off = 0;
        if (valid) {
            const int64_t page =
                clamp_page(a.page_table[(int64_t)b * a.max_pages + (t >> a.ps_shift)], a.num_pages);
            off = page * a.stride_page + (int64_t)(t & ps_mask) * a.stride_token;
            float acc = 0.f;
#pragma unroll 4
            for (int d = 0; d < D; d += 4) {
                const float4 k4 = *(const float4 *)(kp + off + d);
                acc = fmaf(qs[d], k4.x, acc);
                acc = fmaf(qs[d + 1], k4.y, acc);
                acc = fmaf(qs[d + 2], k4.z, acc);
                acc = fmaf(qs[d + 3], k4.w, acc);
            }
            u = acc * a.c;
        }
        const float mnew = fmaxf(m, wave_max(u));
        if (mnew == -INFINITY)
            continue;
        const float alpha = fast_exp2(m - mnew);
        const float p = valid ? fast_exp2(u - mnew) : 0.f;
        l = l * alpha + wave_sum(p);
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            o[i] *= alpha;
        pw[lane] = p;
        offs[lane] = off;
        __syncthreads();
        const int nv = kr.hi - base < 64 ? kr.hi - base : 64;
        for (int i = 0; i < nv; ++i) {
            const float pi = pw[i];
            const float *vr = vp + offs[i];
#pragma unroll
            for (int j = 0; j < VPL; ++j)
                o[j] = fmaf(pi, vr[lane + 64 * j], o[j]);
        }
        __syncthreads();
        m = mnew;
    }
    const float inv = has_keys(l) ? 1.f / l : 0.f;
    float *dst = a.ws_o + (row * a.S + split) * D;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
        dst[lane + 64 * j] = o[j] * inv;
    if (lane == 0)
        a.ws_lse[row * a.S + split] = has_keys(l) ? m + __log2f(l) : -INFINITY;
}

struct MergeArgs {
    const void *q;
    const void *k;
    const void *v;
    int bf16;
    int64_t stride_page, stride_head, stride_token, num_pages;
    const int32_t *page_table;
    int32_t max_pages, ps_shift;
    const int32_t *prefix_len;
    int32_t max_prefix_len;
    const uint64_t *masks;
    int32_t W, B, R, Hq, Hkv, G, D, S;
    float c;
    float *ws_o;     // partials [row][S][D]; the window kernel writes the last slot
    float *ws_lse;
    void *out;
    float *lse2;
};

template <int D, bool BF16>
__device__ inline void load_row(const void *base, int64_t off, int lane, float (&x)[D / 64]) {
#pragma unroll
    for (int j = 0; j < D / 64; ++j) {
        if (BF16)
            x[j] = bf16_bits_to_f32(((const uint16_t *)base)[off + lane * (D / 64) + j]);
        else
            x[j] = ((const float *)base)[off + lane * (D / 64) + j];
    }
}

// Window part and merge: one wave per (request b, row r, head h).  The window
// keys are the set bits j < W of the row's ancestor mask, at logical position
// P + j; unseen window slots are never read.  The window's (o, lse2) is then
// merged with the S prefix partials: lse2 = log2 sum_k 2^lse2_k and
// out = sum_k 2^(lse2_k - lse2) o_k.
template <int D, bool BF16>
__global__ void __launch_bounds__(256) k_window_merge(MergeArgs a) {
    constexpr int VPL = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= (int64_t)a.B * a.R * a.Hq)
        return;
    const int h = (int)(row % a.Hq);
    const int r = (int)((row / a.Hq) % a.R);
    const int b = (int)(row / ((int64_t)a.Hq * a.R));
    const int g = h / a.G;
    float q[VPL];
    load_row<D, BF16>(a.q, row * D, lane, q);
    int P = a.prefix_len[b];
    P = P < 0 ? 0 : (P > a.max_prefix_len ? a.max_prefix_len : P);
    uint64_t msk = a.W > 0 ? a.masks[(int64_t)b * a.R + r] : 0ull;
    if (a.W < 64)
        msk &= (1ull << a.W) - 1ull;
    const int ps_mask = (1 << a.ps_shift) - 1;
    float mw = -INFINITY, lw = 0.f, ow[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j)
        ow[j] = 0.f;
    while (msk) {
        const int j = __ffsll((unsigned long long)msk) - 1;
        msk &= msk - 1;
        const int t = P + j;
        const int64_t page =
            clamp_page(a.page_table[(int64_t)b * a.max_pages + (t >> a.ps_shift)], a.num_pages);
        const int64_t off = page * a.stride_page + (int64_t)g * a.stride_head +
                            (int64_t)(t & ps_mask) * a.stride_token;
        float kx[VPL], vx[VPL];
        load_row<D, BF16>(a.k, off, lane, kx);
        load_row<D, BF16>(a.v, off, lane, vx);
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            dot = fmaf(q[i], kx[i], dot);
        const float u = wave_sum(dot) * a.c;
        const float mnew = fmaxf(mw, u);
        const float alpha = fast_exp2(mw - mnew);
        const float p = fast_exp2(u - mnew);
        lw = lw * alpha + p;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            ow[i] = fmaf(p, vx[i], ow[i] * alpha);
        mw = mnew;
    }
    const float lse_w = has_keys(lw) ? mw + __log2f(lw) : -INFINITY;
    const float *lp = a.ws_lse + row * a.S;
    // max over the parts' lse2, NaN-propagating (a NaN part makes the row NaN)
    float mx = lse_w;
    for (int s = 0; s < a.S; ++s) {
        const float ls = lp[s];
        mx = (ls > mx || ls != ls) ? ls : mx;
    }
    float acc[VPL];
    float res_lse = -INFINITY;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        acc[i] = 0.f;
    if (mx != -INFINITY) {
        float zs = 0.f;
        for (int s = 0; s < a.S; ++s) {
            const float ls = lp[s];
            if (ls == -INFINITY)
                continue;
            const float z = fast_exp2(ls - mx);
            zs += z;
            const float *op = a.ws_o + (row * a.S + s) * D + lane * VPL;
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                acc[i] = fmaf(z, op[i], acc[i]);
        }
        if (lse_w != -INFINITY) {
            const float z = fast_exp2(lse_w - mx);
            const float inv = 1.f / lw;
            zs += z;
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                acc[i] = fmaf(z, ow[i] * inv, acc[i]);
        }
        const float inv = 1.f / zs;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            acc[i] *= inv;
        res_lse = mx + __log2f(zs);
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        if (BF16)
            ((uint16_t *)a.out)[row * D + lane * VPL + i] = f32_to_bf16_bits(acc[i]);
        else
            ((float *)a.out)[row * D + lane * VPL + i] = acc[i];
    }
    if (a.lse2 && lane == 0)
        a.lse2[row] = res_lse;
}


// Window part and merge for bf16 on MFMA.  One workgroup of NW waves per
// (request b, kv head g, group of 32 NW folded rows); a wave owns 32 rows.
// The W window keys of (b, g) (logical positions P .. P + W - 1) are staged
// in LDS, S^T = K_w Q^T and O^T = V_w^T P^T run on v_mfma_f32_32x32x16_bf16
// with each row's ancestor mask applied to the scores, and the window's
// (o, lse2) is merged with the S prefix partials of the row:
// lse2 = log2 sum_k 2^lse2_k, out = sum_k 2^(lse2_k - lse2) o_k.
//
// A window key is shared by every row of the tile, so a non-finite V value
// of a key that a row cannot see would otherwise reach it as 0 * inf.  Such
// values are set to 0 in LDS and their keys flagged; a row that sees a
// flagged key then adds, per channel, the sum of the non-finite values of
// its visible flagged keys to its window output, which is what the exact
// weighted sum gives (positive weights keep infinities and NaN).
template <int D, int NW, bool KV8>
__global__ void __launch_bounds__(64 * NW) k_window_mfma(MergeArgs a) {
    constexpr int KSTEPS = D / 16, DT = D / 32, CH = D / 8, ROWB = D * 2;
    constexpr int THREADS = 64 * NW;
    constexpr int NL = 64 * CH / THREADS;   // bf16 slots per thread and region
    static_assert(64 * CH % THREADS == 0, "slot split");
    __shared__ __attribute__((aligned(16))) char kw[64 * ROWB];
    __shared__ __attribute__((aligned(16))) char vw[64 * ROWB];
    __shared__ uint32_t bad[2];   // keys 0..31, 32..63 with a non-finite V value

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int hl = lane >> 5;
    const int l32 = lane & 31;
    const int M = a.R * a.G;
    const int RGw = (M + 32 * NW - 1) / (32 * NW);
    const int rg = blockIdx.x % RGw;
    const int g = (blockIdx.x / RGw) % a.Hkv;
    const int b = blockIdx.x / (RGw * a.Hkv);
    int P = a.prefix_len[b];
    P = P < 0 ? 0 : (P > a.max_prefix_len ? a.max_prefix_len : P);
    const int W = a.W;
    const int ps_mask = (1 << a.ps_shift) - 1;

    if (tid < 2)
        bad[tid] = 0u;
    if constexpr (KV8) {
        // FP8 E4M3 caches: each thread loads 16-byte chunks (16 values) of
        // K and V, converts them exactly to bf16, zeroes and flags non-finite
        // V values, and writes the bf16 layout below
        constexpr int C8 = D / 16;
        __syncthreads();
        for (int i = tid; i < 64 * C8; i += THREADS) {
            const int key = i / C8, c8 = i % C8;
            int4 k8 = make_int4(0, 0, 0, 0), v8 = make_int4(0, 0, 0, 0);
            if (key < W) {
                const int t = P + key;
                const int64_t page = clamp_page(a.page_table[(int64_t)b * a.max_pages + (t >> a.ps_shift)],
                                                a.num_pages);
                const int64_t off = page * a.stride_page + (int64_t)g * a.stride_head +
                                    (int64_t)(t & ps_mask) * a.stride_token + c8 * 16;
                k8 = *(const int4 *)((const uint8_t *)a.k + off);
                v8 = *(const int4 *)((const uint8_t *)a.v + off);
            }
            int4 kh[2], vh[2];
            fp8x16_to_bf16(k8, kh[0], kh[1]);
            fp8x16_to_bf16(v8, vh[0], vh[1]);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                uint32_t x[4] = {(uint32_t)vh[e].x, (uint32_t)vh[e].y, (uint32_t)vh[e].z, (uint32_t)vh[e].w};
                bool nf = false;
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int hh2 = 0; hh2 < 2; ++hh2)
                        if (((x[q] >> (16 * hh2)) & 0x7F80u) == 0x7F80u) {
                            nf = true;
                            x[q] &= ~(0xFFFFu << (16 * hh2));
                        }
                if (nf)
                    atomicOr(&bad[key >> 5], 1u << (key & 31));
                const int at = key * ROWB + (((2 * c8 + e) ^ swz<D>(key)) * 16);
                *(int4 *)(kw + at) = kh[e];
                *(int4 *)(vw + at) = make_int4((int)x[0], (int)x[1], (int)x[2], (int)x[3]);
            }
        }
    } else {
        // Stage the window keys: key k's 16-byte chunk c sits at LDS byte
        // k * ROWB + 16 (c ^ swz(k)).  Slot i = k * CH + pos of a region is filled
        // by a direct-to-LDS load of chunk pos ^ swz(k); rows of keys >= W are
        // zero.
        int32_t pg[NL];
    #pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int key = (i * THREADS + tid) / CH;
            const int t = P + (key < W ? key : 0);
            pg[i] = key < W ? (int32_t)clamp_page(a.page_table[(int64_t)b * a.max_pages + (t >> a.ps_shift)],
                                                  a.num_pages)
                            : 0;
        }
        const uint32_t kw0 = lds_off(kw), vw0 = lds_off(vw);
    #pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int slot = i * THREADS + tid, key = slot / CH, pos = slot % CH;
            if (key < W) {
                const int t = P + key;
                const int64_t off = (int64_t)pg[i] * a.stride_page + (int64_t)g * a.stride_head +
                                    (int64_t)(t & ps_mask) * a.stride_token + ((pos ^ swz<D>(key)) * 8);
                const uint32_t at = (uint32_t)((i * THREADS + w * 64) * 16);
                dma_load16((const uint16_t *)a.k + off, __builtin_amdgcn_readfirstlane(kw0 + at));
                dma_load16((const uint16_t *)a.v + off, __builtin_amdgcn_readfirstlane(vw0 + at));
            } else {
                *(int4 *)(kw + slot * 16) = make_int4(0, 0, 0, 0);
                *(int4 *)(vw + slot * 16) = make_int4(0, 0, 0, 0);
            }
        }
    }
    const int m = rg * 32 * NW + w * 32 + l32;   // this lane's folded row
    const bool ok = m < M;
    const int r = ok ? m / a.G : 0, hh = ok ? m % a.G : 0;
    const int64_t row = ((int64_t)b * a.R + r) * a.Hq + (int64_t)g * a.G + hh;
    bf16x8 qv[KSTEPS];
    {
        const uint16_t *qp = (const uint16_t *)a.q + row * D + 8 * hl;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            int4 v4 = ok ? *(const int4 *)(qp + 16 * kk) : make_int4(0, 0, 0, 0);
            qv[kk] = __builtin_bit_cast(bf16x8, v4);
        }
    }
    uint64_t rmask = ok && W > 0 ? a.masks[(int64_t)b * a.R + r] : 0ull;
    if (W < 64)
        rmask &= (1ull << W) - 1ull;
    wait_vmcnt<0>();
    __syncthreads();
    // non-finite V values: zero them in LDS and flag their keys
#pragma unroll
    for (int i = 0; i < (KV8 ? 0 : NL); ++i) {
        const int slot = i * THREADS + tid, key = slot / CH;
        if (key < W) {
            uint4 u = *(const uint4 *)(vw + slot * 16);
            uint32_t x[4] = {u.x, u.y, u.z, u.w};
            bool nf = false;
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int hh2 = 0; hh2 < 2; ++hh2)
                    if (((x[e] >> (16 * hh2)) & 0x7F80u) == 0x7F80u) {
                        nf = true;
                        x[e] &= ~(0xFFFFu << (16 * hh2));
                    }
            if (nf) {
                *(uint4 *)(vw + slot * 16) = make_uint4(x[0], x[1], x[2], x[3]);
                atomicOr(&bad[key >> 5], 1u << (key & 31));
            }
        }
    }
    __syncthreads();

    // window scores, exact row max, weights and O over the (at most two)
    // 32-key blocks
    const int nkb = (W + 31) / 32;
    f32x16 s[2];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        if (kb >= nkb)
            break;
        const int krow = kb * 32 + l32;
        const int ksw = swz<D>(krow);
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            const bf16x8 ka = *(const bf16x8 *)(kw + krow * ROWB + (((2 * kk + hl) ^ ksw) * 16));
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qv[kk], kk ? s[kb] : f32x16{}, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int j = kb * 32 + 8 * (e >> 2) + 4 * hl + (e & 3);
            if (!((rmask >> j) & 1ull))
                s[kb][e] = -INFINITY;
            mx = fmaxf(mx, s[kb][e]);
        }
    }
    mx = pair_max(mx) * a.c;
    const float mu = mx == -INFINITY ? 0.f : mx;
    f32x16 o[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            o[t][e] = 0.f;
    float l = 0.f;
    const int G16 = lane >> 4, a4 = lane & 3, j4 = (lane >> 2) & 3;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        if (kb >= nkb)
            break;
        // weights split into a bf16 head and a bf16 remainder: the window
        // has few keys, so their rounding would not average out
        bf16x8 pb[2], pr[2];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float p = fast_exp2(fmaf(s[kb][e], a.c, -mu));
            const __bf16 ph = (__bf16)p;
            pb[e >> 3][e & 7] = ph;
            pr[e >> 3][e & 7] = (__bf16)(p - (float)ph);
            l += p;
        }
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            const int d0 = ((G16 & 1) ? D / 2 : 0) + 16 * t + 4 * a4;
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                i16x4 half[2];
#pragma unroll
                for (int hr = 0; hr < 2; ++hr) {
                    const int key = kb * 32 + cc * 16 + hr * 8 + 4 * (G16 >> 1) + j4;
                    const char *p = vw + key * ROWB + (((d0 >> 3) ^ swz<D>(key)) * 16) + (a4 & 1) * 8;
                    half[hr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)p);
                }
                struct {
                    i16x4 lo, hi;
                } pair{half[0], half[1]};
                const bf16x8 va = __builtin_bit_cast(bf16x8, pair);
                o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[cc], o[t], 0, 0, 0);
                o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pr[cc], o[t], 0, 0, 0);
            }
        }
    }
    const float lt = pair_sum(l);
    const float lse_w = has_keys(lt) ? mu + __log2f(lt) : -INFINITY;
    const float inv_w = has_keys(lt) ? 1.f / lt : 0.f;
    // lane value o[t][e] is channel d(t, e) of row m
    auto chan = [&](int t, int e) {
        return ((e >> 3) ? D / 2 : 0) + 16 * t + 8 * ((e >> 2) & 1) + 4 * hl + (e & 3);
    };
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            o[t][e] *= inv_w;
    // visible keys with non-finite V values (rare): add those values
    uint64_t vbad = rmask & (((uint64_t)bad[1] << 32) | bad[0]);
    if (__ballot(vbad != 0ull)) {
        while (vbad) {
            const int j = __ffsll((unsigned long long)vbad) - 1;
            vbad &= vbad - 1;
            const int t_ = P + j;
            const int64_t page =
                clamp_page(a.page_table[(int64_t)b * a.max_pages + (t_ >> a.ps_shift)], a.num_pages);
            const int64_t vo = page * a.stride_page + (int64_t)g * a.stride_head +
                               (int64_t)(t_ & ps_mask) * a.stride_token;
#pragma unroll
            for (int t = 0; t < DT; ++t)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float x = KV8 ? fp8_to_f32(((const uint8_t *)a.v)[vo + chan(t, e)])
                                        : bf16_bits_to_f32(((const uint16_t *)a.v)[vo + chan(t, e)]);
                    if (!(fabsf(x) < INFINITY))
                        o[t][e] += x;
                }
        }
    }
    if (!ok)
        return;
    if (a.S == 2) {
        // a single prefix partial: merge it here (NaN-propagating max) and
        // write the row's output
        const float lp = a.ws_lse[row * 2];
        const float mall = (lp > lse_w || lp != lp) ? lp : lse_w;
        float res_lse = -INFINITY;
        const float *op = a.ws_o + row * 2 * D;
        if (mall != -INFINITY) {
            const float zp = lp != -INFINITY ? fast_exp2(lp - mall) : 0.f;
            const float zw = lse_w != -INFINITY ? fast_exp2(lse_w - mall) : 0.f;
            const float inv = 1.f / (zp + zw);
#pragma unroll
            for (int t = 0; t < DT; ++t)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const float4 v4 = *(const float4 *)(op + chan(t, 4 * q4));
                    const float pv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float wv = lse_w != -INFINITY ? zw * o[t][4 * q4 + e] : 0.f;
                        o[t][4 * q4 + e] = (lp != -INFINITY ? fmaf(zp, pv[e], wv) : wv) * inv;
                    }
                }
            res_lse = mall + __log2f(zp + zw);
        } else {
#pragma unroll
            for (int t = 0; t < DT; ++t)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    o[t][e] = 0.f;
        }
        uint16_t *out = (uint16_t *)a.out + row * D;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const uint32_t lo = f32_to_bf16_bits(o[t][4 * q4]) |
                                    ((uint32_t)f32_to_bf16_bits(o[t][4 * q4 + 1]) << 16);
                const uint32_t hi = f32_to_bf16_bits(o[t][4 * q4 + 2]) |
                                    ((uint32_t)f32_to_bf16_bits(o[t][4 * q4 + 3]) << 16);
                *(uint2 *)(out + chan(t, 4 * q4)) = make_uint2(lo, hi);
            }
        if (a.lse2 && hl == 0)
            a.lse2[row] = res_lse;
        return;
    }
    // the window's partial goes to the last slot of the row
    float *dst = a.ws_o + (row * a.S + (a.S - 1)) * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            *(float4 *)(dst + chan(t, 4 * q4)) =
                make_float4(o[t][4 * q4], o[t][4 * q4 + 1], o[t][4 * q4 + 2], o[t][4 * q4 + 3]);
    if (hl == 0)
        a.ws_lse[row * a.S + (a.S - 1)] = lse_w;
}

__device__ inline float nan_max(float x, float y) {
    return (x != x || y != y) ? __builtin_nanf("") : fmaxf(x, y);
}

// Merge of the S partials of a row (prefix splits and the window, bf16
// path), lanes over channels.  SPL waves share a row: wave w takes partials
// w, w + SPL, ...; with SPL = 1 a workgroup merges four rows, otherwise one.
// lse2 = log2 sum_k 2^lse2_k, out = sum_k 2^(lse2_k - lse2) o_k; the max is
// NaN-propagating, so a NaN partial makes the row NaN.  A wave loads up to
// 16 partials per round, their values and LSEs all in flight before the
// first use, and weighs them against the largest LSE it has seen (rescaling
// when a later round raises it); the waves' sums then combine in LDS against
// the row's max.  A row whose partials fit one round thus costs one load
// round trip.
template <int D, int SPL>
__global__ void __launch_bounds__(256 * (SPL > 4 ? SPL / 4 : 1)) k_merge(MergeArgs a) {
    constexpr int VPL = D / 64;
    constexpr int RPW = SPL >= 4 ? 1 : 4 / SPL;   // rows per workgroup
    constexpr int MB = 16;
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int part = wv % SPL;
    const int64_t row = (int64_t)blockIdx.x * RPW + wv / SPL;
    // (with SPL > 1 the grid holds exactly one workgroup per row, so this
    // exit never splits a workgroup before its barrier)
    if (row >= (int64_t)a.B * a.R * a.Hq)
        return;
    const float *lp = a.ws_lse + row * a.S;
    const float *op = a.ws_o + row * a.S * D + lane * VPL;
    float acc[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        acc[i] = 0.f;
    float m = -INFINITY, zs = 0.f;
    for (int s0 = part; s0 < a.S; s0 += MB * SPL) {
        float x[MB][VPL], ls[MB];
#pragma unroll
        for (int j = 0; j < MB; ++j) {
            const int sj = s0 + j * SPL;
            const bool in = sj < a.S;
            ls[j] = in ? lp[sj] : -INFINITY;
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                x[j][i] = in ? op[(int64_t)sj * D + i] : 0.f;
        }
        float mn = m;
#pragma unroll
        for (int j = 0; j < MB; ++j)
            mn = nan_max(mn, ls[j]);
        if (mn != m) {   // (also when either is NaN)
            const float sc = m == -INFINITY ? 0.f : fast_exp2(m - mn);
            zs *= sc;
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                acc[i] *= sc;
            m = mn;
        }
        if (m == -INFINITY)
            continue;
#pragma unroll
        for (int j = 0; j < MB; ++j) {
            const float z = ls[j] != -INFINITY ? fast_exp2(ls[j] - m) : 0.f;
            zs += z;
            if (ls[j] != -INFINITY) {
#pragma unroll
                for (int i = 0; i < VPL; ++i)
                    acc[i] = fmaf(z, x[j][i], acc[i]);
            }
        }
    }
    if constexpr (SPL > 1) {
        __shared__ float red[SPL][D + 2];
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            red[part][lane * VPL + i] = acc[i];
        if (lane == 0) {
            red[part][D] = zs;
            red[part][D + 1] = m;
        }
        __syncthreads();
        if (part != 0)
            return;
        float mw[SPL];
        m = -INFINITY;
#pragma unroll
        for (int w = 0; w < SPL; ++w) {
            mw[w] = red[w][D + 1];
            m = nan_max(m, mw[w]);
        }
        zs = 0.f;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            acc[i] = 0.f;
        if (m != -INFINITY) {
#pragma unroll
            for (int w = 0; w < SPL; ++w) {
                const float f = mw[w] == -INFINITY ? 0.f : fast_exp2(mw[w] - m);
                zs = fmaf(f, red[w][D], zs);
#pragma unroll
                for (int i = 0; i < VPL; ++i)
                    acc[i] = fmaf(f, red[w][lane * VPL + i], acc[i]);
            }
        }
    }
    float res_lse = -INFINITY;
    if (m != -INFINITY) {
        const float inv = 1.f / zs;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            acc[i] *= inv;
        res_lse = m + __log2f(zs);
    }
    uint16_t *dst = (uint16_t *)a.out + row * D + lane * VPL;
    if (VPL == 2)
        *(uint32_t *)dst = f32_to_bf16_bits(acc[0]) | ((uint32_t)f32_to_bf16_bits(acc[VPL - 1]) << 16);
    else
        dst[0] = f32_to_bf16_bits(acc[0]);
    if (a.lse2 && lane == 0)
        a.lse2[row] = res_lse;
}

// ---------------------------------------------------------------------------
// host plan
// ---------------------------------------------------------------------------

struct Plan {
    bool mfma;
    int NT, NRB, NKS, RG, n_split, kps, S;
    size_t o_bytes, lse_off, bytes;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Plan make_plan(tav_dtype dtype, int B, int R, int Hq, int Hkv, int D, int max_prefix_len,
               int prefix_window, int page_size) {
    Plan p{};
    const int G = Hq / Hkv;
    const long long M = (long long)R * G;
    const int max_vis = prefix_window > 0 && prefix_window < max_prefix_len ? prefix_window
                                                                            : max_prefix_len;
    if (dtype == TAV_BF16 || dtype == TAV_FP8_E4M3) {
        p.mfma = true;
        p.NT = 1;
        if (M <= 32) {
            p.NRB = 1;
            p.NKS = dtype == TAV_BF16 ? 2 : 4;
        } else if (M <= 64) {
            p.NRB = 2;
            p.NKS = 4;
        } else if (M <= 128 || (dtype == TAV_FP8_E4M3 && D != 128)) {
            // (the pipelined kernel's FP8 path takes 128-channel heads; other
            // FP8 widths run 128-row groups here)
            p.NRB = 4;
            p.NKS = 2;
        } else {
            p.NRB = 8;
            p.NKS = 1;
        }
        const int rows_wg = p.NRB * 32;
        p.RG = (int)((M + rows_wg - 1) / rows_wg);
        const int SK = p.NRB == 8 ? kPipeStageKeys : 32 * p.NKS;
        const long long base = (long long)B * Hkv * p.RG;
        int n = base > 0 ? (int)((256 + base - 1) / base) : 1;
        const int by_stages = max_vis / (4 * SK);            // >= 4 stages per split
        n = n < by_stages ? n : by_stages;
        n = n < 1 ? 1 : n;
        // keys per split: a whole number of stages whose page-table slice
        // fits the LDS slice, also with the 8 keys below the split start that
        // a stage may begin with and the 64 window keys a fused call appends
        // ((kps + 72) / page_size + 2 entries at most)
        int kps;
        for (;;) {
            kps = (max_vis + n - 1) / n;
            kps = ((kps + SK - 1) / SK) * SK;
            if (kps < SK)
                kps = SK;
            if ((long long)(kps + 72) / page_size + 2 <= kPtMax)
                break;
            ++n;
        }
        p.kps = kps;
        p.n_split = max_vis > 0 ? (max_vis + kps - 1) / kps : 1;
        p.S = p.n_split + 1;   // one partial per split (the key subsets combined); the
                               // last slot holds the window partial
    } else {
        p.mfma = false;
        p.NT = p.NRB = p.NKS = p.RG = 1;
        const long long rows = (long long)B * R * Hq;
        int n = rows > 0 ? (int)((1024 + rows - 1) / rows) : 1;
        const int by_keys = max_vis / 256;
        n = n < by_keys ? n : by_keys;
        n = n < 1 ? 1 : n;
        int kps = (max_vis + n - 1) / n;
        p.kps = kps < 1 ? 1 : kps;
        p.n_split = max_vis > 0 ? (max_vis + p.kps - 1) / p.kps : 1;
        p.S = p.n_split;
    }
    const size_t rows = (size_t)B * R * Hq;
    p.o_bytes = align256(rows * p.S * D * sizeof(float));
    p.lse_off = p.o_bytes;
    p.bytes = p.o_bytes + align256(rows * p.S * sizeof(float));
    if (p.bytes < 256)
        p.bytes = 256;  // a valid size is never 0
    return p;
}

bool shape_ok(tav_dtype dtype, int B, int R, int Hq, int Hkv, int D, int max_prefix_len,
              int prefix_window, int page_size, tav::Checks *c) {
    tav::Checks local;
    tav::Checks &k = c ? *c : local;
    using tav::str;
    TAV_NEED(k, dtype == TAV_F32 || dtype == TAV_BF16 || dtype == TAV_FP8_E4M3, TAV_ERR_UNSUPPORTED,
             "dtype must be TAV_F32, TAV_BF16 or TAV_FP8_E4M3, got " + str(dtype));
    TAV_NEED(k, B >= 0, TAV_ERR_INVALID_ARG, "B must be >= 0, got " + str(B));
    TAV_NEED(k, R >= 1 && R <= 64, TAV_ERR_INVALID_ARG, "R must be in [1, 64], got " + str(R));
    TAV_NEED(k, Hq >= 1 && Hkv >= 1, TAV_ERR_INVALID_ARG,
             "Hq and Hkv must be >= 1, got " + str(Hq) + ", " + str(Hkv));
    TAV_NEED(k, Hkv >= 1 && Hq % Hkv == 0, TAV_ERR_INVALID_ARG,
             "Hq must be a multiple of Hkv, got " + str(Hq) + " % " + str(Hkv));
    TAV_NEED(k, D == 64 || D == 128, TAV_ERR_UNSUPPORTED, "D must be 64 or 128, got " + str(D));
    TAV_NEED(k, max_prefix_len >= 0, TAV_ERR_INVALID_ARG,
             "max_prefix_len must be >= 0, got " + str(max_prefix_len));
    TAV_NEED(k, prefix_window >= 0, TAV_ERR_INVALID_ARG,
             "prefix_window must be >= 0, got " + str(prefix_window));
    TAV_NEED(k, tav::is_pow2(page_size) && page_size <= 1024, TAV_ERR_UNSUPPORTED,
             "page_size must be a power of two in [1, 1024], got " + str(page_size));
    TAV_NEED(k, (long long)B * R * Hq <= (1LL << 30), TAV_ERR_INVALID_ARG,
             "B * R * Hq is too large");
    return k.status == TAV_OK;
}

template <int D, int NRB, int NKS, bool KV8>
void launch_mfma(const Plan &p, const PrefixArgs &a, hipStream_t s) {
    const unsigned grid = (unsigned)((long long)a.B * a.Hkv * p.RG * p.n_split);
    hipLaunchKernelGGL((k_prefix_mfma<D, NRB, NKS, KV8>), dim3(grid), dim3(64 * NRB * NKS), 0, s, a);
}

template <int D, bool KV8>
void launch_mfma_d(const Plan &p, const PrefixArgs &a, hipStream_t s) {
    if constexpr (!KV8) {
        if (p.NRB == 1 && p.NKS == 2) {
            launch_mfma<D, 1, 2, KV8>(p, a, s);
            return;
        }
    }
    if (p.NRB == 1)
        launch_mfma<D, 1, 4, KV8>(p, a, s);
    else if (p.NRB == 2)
        launch_mfma<D, 2, 4, KV8>(p, a, s);
    else if (p.NRB == 4)
        launch_mfma<D, 4, 2, KV8>(p, a, s);
    else if constexpr (!KV8 || D == 128) {
        const unsigned grid = (unsigned)((long long)a.B * a.Hkv * p.RG * p.n_split);
        hipLaunchKernelGGL((k_prefix_mfma_pipe<D, kPipeStageKeys, KV8>), dim3(grid), dim3(512), 0, s, a);
    }
}

// Arguments of one tree_attention call after validation.
struct Call {
    Plan p;
    PrefixArgs a;
    MergeArgs m;
    int D;
    bool bf16;   // bf16 query and output (bf16 or FP8 K/V)
    bool kv8;    // FP8 E4M3 K/V
    bool fused;  // the prefix launch also takes the window keys and writes the output
};

// Validates every argument (all failures are reported together) and builds
// the launch arguments.  `phase`: 1 = prefix only, 2 = window + merge only,
// 3 = both.
tav_status prepare(const char *fn, int phase, Call &call, const void *q, const void *k_cache,
                   const void *v_cache, tav_dtype dtype, int64_t stride_page,
                   int64_t stride_head, int64_t stride_token, int64_t num_pages,
                   const int32_t *page_table, int32_t max_pages, int32_t page_size,
                   const int32_t *prefix_len, int32_t max_prefix_len, int32_t prefix_window,
                   const uint64_t *masks, int32_t W, int32_t B, int32_t R, int32_t Hq,
                   int32_t Hkv, int32_t D, float sm_scale, void *out, float *lse2,
                   void *workspace, size_t workspace_bytes) {
    using tav::str;
    tav::Checks c;
    shape_ok(dtype, B, R, Hq, Hkv, D, max_prefix_len, prefix_window, page_size, &c);
    TAV_NEED(c, W >= 0 && W <= 64, TAV_ERR_INVALID_ARG, "W must be in [0, 64], got " + str(W));
    TAV_NEED(c, max_pages >= 1, TAV_ERR_INVALID_ARG,
             "max_pages must be >= 1, got " + str(max_pages));
    TAV_NEED(c, (long long)max_pages * page_size >= (long long)max_prefix_len + W,
             TAV_ERR_INVALID_ARG,
             "max_pages * page_size (" + str((long long)max_pages * page_size) +
                 ") must cover max_prefix_len + W (" + str((long long)max_prefix_len + W) + ")");
    TAV_NEED(c, num_pages >= 1, TAV_ERR_INVALID_ARG,
             "num_pages must be >= 1, got " + str(num_pages));
    TAV_NEED(c, std::isfinite(sm_scale), TAV_ERR_INVALID_ARG, "sm_scale must be finite");
    const int esz = dtype == TAV_F32 ? 4 : (dtype == TAV_FP8_E4M3 ? 1 : 2);   // K/V element bytes
    TAV_NEED(c, stride_page >= 0 && stride_head >= 0 && stride_token >= 0, TAV_ERR_INVALID_ARG,
             "strides must be >= 0");
    TAV_NEED(c, (stride_page * esz) % 16 == 0 && (stride_head * esz) % 16 == 0 &&
                 (stride_token * esz) % 16 == 0,
             TAV_ERR_UNSUPPORTED, "K/V strides must be multiples of 16 bytes");
    TAV_NEED(c, stride_token * esz < (1LL << 27), TAV_ERR_UNSUPPORTED,
             "stride_token must be below 2^27 bytes");
    if (B > 0) {
        TAV_NEED(c, q && k_cache && v_cache, TAV_ERR_INVALID_ARG,
                 "q, k_cache and v_cache must be set");
        TAV_NEED(c, page_table && prefix_len, TAV_ERR_INVALID_ARG,
                 "page_table and prefix_len must be set");
        if (phase & 2) {
            TAV_NEED(c, W == 0 || masks, TAV_ERR_INVALID_ARG, "masks is NULL");
            TAV_NEED(c, out, TAV_ERR_INVALID_ARG, "out is NULL");
        }
        TAV_NEED(c, workspace, TAV_ERR_WORKSPACE, "workspace is NULL");
        const uintptr_t any_addr =
            (uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out;
        TAV_NEED(c, (any_addr & 15) == 0, TAV_ERR_UNSUPPORTED,
                 "q, k_cache, v_cache and out must be 16-byte aligned");
        TAV_NEED(c, ((uintptr_t)workspace & 255) == 0, TAV_ERR_WORKSPACE,
                 "workspace must be 256-byte aligned");
    }
    if (c.status == TAV_OK) {
        call.p = make_plan(dtype, B, R, Hq, Hkv, D, max_prefix_len, prefix_window, page_size);
        TAV_NEED(c, workspace_bytes >= call.p.bytes, TAV_ERR_WORKSPACE,
                 "workspace has " + str((long long)workspace_bytes) + " bytes, needs " +
                     str((long long)call.p.bytes));
    }
    if (c.status != TAV_OK)
        return tav::finish(fn, c);

    const Plan &p = call.p;
    const float scale = sm_scale > 0.f ? sm_scale : 1.f / std::sqrt((float)D);
    PrefixArgs &a = call.a;
    a = PrefixArgs{};
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.stride_page = stride_page;
    a.stride_head = stride_head;
    a.stride_token = stride_token;
    a.num_pages = num_pages;
    a.page_table = page_table;
    a.max_pages = max_pages;
    a.ps_shift = tav::ilog2(page_size);
    a.prefix_len = prefix_len;
    a.max_prefix_len = max_prefix_len;
    a.prefix_window = prefix_window;
    a.B = B;
    a.R = R;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.M = R * a.G;
    a.RG = p.RG;
    a.n_split = p.n_split;
    a.kps = p.kps;
    a.S = p.S;
    a.c = scale * kLog2e;
    a.ws_o = (float *)workspace;
    a.ws_lse = (float *)((char *)workspace + p.lse_off);

    MergeArgs &m = call.m;
    m = MergeArgs{};
    m.q = q;
    m.k = k_cache;
    m.v = v_cache;
    m.bf16 = dtype != TAV_F32;
    m.stride_page = stride_page;
    m.stride_head = stride_head;
    m.stride_token = stride_token;
    m.num_pages = num_pages;
    m.page_table = page_table;
    m.max_pages = max_pages;
    m.ps_shift = a.ps_shift;
    m.prefix_len = prefix_len;
    m.max_prefix_len = max_prefix_len;
    m.masks = masks;
    m.W = W;
    m.B = B;
    m.R = R;
    m.Hq = Hq;
    m.Hkv = Hkv;
    m.G = a.G;
    m.D = D;
    m.S = p.S;
    m.c = a.c;
    m.ws_o = a.ws_o;
    m.ws_lse = a.ws_lse;
    m.out = out;
    m.lse2 = lse2;
    call.D = D;
    call.bf16 = dtype != TAV_F32;
    call.kv8 = dtype == TAV_FP8_E4M3;
    // One split on the pipelined kernel over bf16 K/V, with the masks and
    // the output given: the prefix launch takes the window keys too and
    // writes the output, and the window-and-merge phase launches nothing.
    // Both phases decide it from their (identical) arguments.
    call.fused = dtype == TAV_BF16 && p.mfma && (p.NRB == 8 || p.NRB == 1) && p.n_split == 1 &&
                 out != nullptr && (W == 0 || masks != nullptr);
    if (call.fused) {
        a.fuse = 1;
        a.W = W;
        a.masks = masks;
        a.out = out;
        a.lse2 = lse2;
    }
    return TAV_OK;
}

void launch_prefix(const Call &c, hipStream_t s) {
    const Plan &p = c.p;
    if (p.mfma) {
        if (c.D == 128)
            c.kv8 ? launch_mfma_d<128, true>(p, c.a, s) : launch_mfma_d<128, false>(p, c.a, s);
        else
            c.kv8 ? launch_mfma_d<64, true>(p, c.a, s) : launch_mfma_d<64, false>(p, c.a, s);
    } else {
        const unsigned grid = (unsigned)((long long)c.a.B * c.a.R * c.a.Hq * p.n_split);
        if (c.D == 128)
            hipLaunchKernelGGL(k_prefix_f32<128>, dim3(grid), dim3(64), 0, s, c.a);
        else
            hipLaunchKernelGGL(k_prefix_f32<64>, dim3(grid), dim3(64), 0, s, c.a);
    }
}

template <int D, int NW, bool KV8>
void launch_window_mfma(const MergeArgs &m, hipStream_t s) {
    const int M = m.R * m.G;
    const unsigned grid = (unsigned)((long long)m.B * m.Hkv * ((M + 32 * NW - 1) / (32 * NW)));
    hipLaunchKernelGGL((k_window_mfma<D, NW, KV8>), dim3(grid), dim3(64 * NW), 0, s, m);
}

template <int D, bool KV8>
void launch_window_mfma_d(const MergeArgs &m, hipStream_t s) {
    const int M = m.R * m.G;
    if (M <= 32)
        launch_window_mfma<D, 1, KV8>(m, s);
    else if (M <= 64)
        launch_window_mfma<D, 2, KV8>(m, s);
    else
        launch_window_mfma<D, 4, KV8>(m, s);
}

// The bf16 merge: one wave per row up to 16 partials (one round of loads),
// else 4 or 8 waves per row, so that each wave's share fits one round up to
// 128 partials.
template <int D>
void launch_merge_d(const MergeArgs &m, hipStream_t s) {
    const long long rows = (long long)m.B * m.R * m.Hq;
    if (m.S <= 16)
        hipLaunchKernelGGL((k_merge<D, 1>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, m);
    else if (m.S <= 64)
        hipLaunchKernelGGL((k_merge<D, 4>), dim3((unsigned)rows), dim3(256), 0, s, m);
    else
        hipLaunchKernelGGL((k_merge<D, 8>), dim3((unsigned)rows), dim3(512), 0, s, m);
}

void launch_merge(const Call &c, hipStream_t s) {
    const MergeArgs &m = c.m;
    const unsigned grid = (unsigned)(((long long)m.B * m.R * m.Hq + 3) / 4);
    if (c.bf16) {
        // with a single prefix partial the window kernel writes the output
        if (c.D == 128) {
            c.kv8 ? launch_window_mfma_d<128, true>(m, s) : launch_window_mfma_d<128, false>(m, s);
            if (m.S > 2)
                launch_merge_d<128>(m, s);
        } else {
            c.kv8 ? launch_window_mfma_d<64, true>(m, s) : launch_window_mfma_d<64, false>(m, s);
            if (m.S > 2)
                launch_merge_d<64>(m, s);
        }
        return;
    }
    if (c.D == 128) {
        if (c.bf16)
            hipLaunchKernelGGL((k_window_merge<128, true>), dim3(grid), dim3(256), 0, s, m);
        else
            hipLaunchKernelGGL((k_window_merge<128, false>), dim3(grid), dim3(256), 0, s, m);
    } else {
        if (c.bf16)
            hipLaunchKernelGGL((k_window_merge<64, true>), dim3(grid), dim3(256), 0, s, m);
        else
            hipLaunchKernelGGL((k_window_merge<64, false>), dim3(grid), dim3(256), 0, s, m);
    }
}

}  // namespace

extern "C" size_t tree_attention_workspace_size(tav_dtype dtype, int32_t B, int32_t R, int32_t Hq,
                                                int32_t Hkv, int32_t D, int32_t max_prefix_len,
                                                int32_t prefix_window, int32_t page_size) {
    if (!shape_ok(dtype, B, R, Hq, Hkv, D, max_prefix_len, prefix_window, page_size, nullptr))
        return 0;
    return make_plan(dtype, B, R, Hq, Hkv, D, max_prefix_len, prefix_window, page_size).bytes;
}

#define TAV_ATTN_PARAMS                                                                         \
    const void *q, const void *k_cache, const void *v_cache, tav_dtype dtype,                   \
        int64_t stride_page, int64_t stride_head, int64_t stride_token, int64_t num_pages,     \
        const int32_t *page_table, int32_t max_pages, int32_t page_size,                        \
        const int32_t *prefix_len, int32_t max_prefix_len, int32_t prefix_window,              \
        const uint64_t *masks, int32_t W, int32_t B, int32_t R, int32_t Hq, int32_t Hkv,       \
        int32_t D, float sm_scale, void *out, float *lse2, void *workspace,                     \
        size_t workspace_bytes, void *stream
#define TAV_ATTN_ARGS                                                                           \
    q, k_cache, v_cache, dtype, stride_page, stride_head, stride_token, num_pages, page_table,  \
        max_pages, page_size, prefix_len, max_prefix_len, prefix_window, masks, W, B, R, Hq,    \
        Hkv, D, sm_scale, out, lse2, workspace, workspace_bytes

static tav_status run_phases(const char *fn, int phase, TAV_ATTN_PARAMS) {
    Call call;
    const tav_status st = prepare(fn, phase, call, TAV_ATTN_ARGS);
    if (st != TAV_OK || B == 0)
        return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (phase & 1) {
        launch_prefix(call, s);
        const tav_status e = tav::launched(fn);
        if (e != TAV_OK)
            return e;
    }
    if ((phase & 2) && !call.fused)
        launch_merge(call, s);
    return tav::launched(fn);
}

extern "C" tav_status tree_attention(TAV_ATTN_PARAMS) {
    return run_phases("tree_attention", 3, TAV_ATTN_ARGS, stream);
}

extern "C" tav_status tree_attention_prefix(TAV_ATTN_PARAMS) {
    return run_phases("tree_attention_prefix", 1, TAV_ATTN_ARGS, stream);
}

extern "C" tav_status tree_attention_window_merge(TAV_ATTN_PARAMS) {
    return run_phases("tree_attention_window_merge", 2, TAV_ATTN_ARGS, stream);
}

// ---------------------------------------------------------------------------
// allocation-free variant: the partials live in a fixed device array
// ---------------------------------------------------------------------------

namespace {

// One copy per GPU the library runs on, held until the process ends.  In
// host code `scratch` only names the symbol; its device address on each GPU
// comes from hipGetSymbolAddress with that GPU current.
constexpr size_t kScratchBytes = TAV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the GPU that runs `stream` (the current
// device for the null stream), resolved on the first call for that GPU.
tav_status scratch_on(const char *fn, hipStream_t stream, void **ptr) {
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        tav::set_error(fn, std::string("cannot tell the stream's device: ") +
                               (e != hipSuccess ? hipGetErrorString(e) : "ordinal out of range"));
        return TAV_ERR_HIP;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev)
            e = hipSetDevice(dev);
        void *p = nullptr;
        if (e == hipSuccess)
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur >= 0 && cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            e = e == hipSuccess ? e2 : e;
        }
        if (e != hipSuccess || !p) {
            tav::set_error(fn, std::string("cannot resolve the static scratch array: ") +
                                   (e != hipSuccess ? hipGetErrorString(e) : "null address"));
            return TAV_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return TAV_OK;
}

}  // namespace

extern "C" tav_status tree_attention_noalloc(
    const void *q, const void *k_cache, const void *v_cache, tav_dtype dtype, int64_t stride_page,
    int64_t stride_head, int64_t stride_token, int64_t num_pages, const int32_t *page_table,
    int32_t max_pages, int32_t page_size, const int32_t *prefix_len, int32_t max_prefix_len,
    int32_t prefix_window, const uint64_t *masks, int32_t W, int32_t B, int32_t R, int32_t Hq,
    int32_t Hkv, int32_t D, float sm_scale, void *out, float *lse2, void *stream) {
    const char *fn = "tree_attention_noalloc";
    tav::Checks c;
    if (shape_ok(dtype, B, R, Hq, Hkv, D, max_prefix_len, prefix_window, page_size, &c)) {
        const size_t need =
            make_plan(dtype, B, R, Hq, Hkv, D, max_prefix_len, prefix_window, page_size).bytes;
        TAV_NEED(c, need <= kScratchBytes, TAV_ERR_WORKSPACE,
                 "this shape needs " + tav::str((long long)need) +
                     " bytes of partials, more than the static scratch array holds (" +
                     tav::str((long long)kScratchBytes) +
                     "); call tree_attention with a workspace instead");
    }
    if (c.status != TAV_OK)
        return tav::finish(fn, c);
    void *ws = nullptr;
    if (B > 0) {
        const tav_status st = scratch_on(fn, reinterpret_cast<hipStream_t>(stream), &ws);
        if (st != TAV_OK)
            return st;
    }
    return run_phases(fn, 3, q, k_cache, v_cache, dtype, stride_page, stride_head, stride_token,
                      num_pages, page_table, max_pages, page_size, prefix_len, max_prefix_len,
                      prefix_window, masks, W, B, R, Hq, Hkv, D, sm_scale, out, lse2, ws,
                      kScratchBytes, stream);
}
