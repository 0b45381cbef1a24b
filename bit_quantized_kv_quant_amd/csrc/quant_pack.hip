// 2-bit asymmetric min/max quantise-and-pack of the kept tokens.
//
// Method: gptget.net summary of arXiv 2411.18077, sections 方法论 / 方法详解
// (2-bit KV quantisation; keys quantised per channel, values per token; a
// compact cache layout).  Group rule of this library, in IEEE fp32 with
// round-half-even and the stored fp16 parameters:
//   s = fp16(fl32(max - min) / 3), z = fp16(min),
//   code = s == 0 ? 0 : clamp(rint(fl32(x - z) / s), 0, 3)
// The file is compiled with -ffp-contract=off so no multiply-add is fused and
// the divide by 3 stays correctly rounded; the codes come from exact threshold
// tests (code_of: comparisons with exact multiples of s) and match a
// plain IEEE evaluation of the rule bit for bit.
// Inputs are finite (-fno-honor-nans: min / max need no NaN handling).
//
// HBM-bound gather: each kept row is read once, each packed byte written once.
// Keys and values of a token group are packed by the two waves of one
// workgroup.  A wave loads its group's 32 rows as whole-row 16-byte chunks
// (every load instruction covers complete rows), derives the group parameters
// with cross-lane reductions (keys: a reduce-scatter over the lanes holding the
// same channels, parameters computed once per channel and handed back; values:
// DPP over the lanes of a 32-channel group), builds the 2-bit codes a bit at a
// time from the comparison masks, and writes them through a small LDS staging
// area so that every global store is a whole 16-byte piece of the packed
// layout.
#include <type_traits>

#include "common.h"
#include "kernels.h"

#pragma clang fp contract(off)

namespace minikv {
namespace {

struct Pair { float a, b; };

template <typename T> __device__ __forceinline__ Pair load_pair(const T* row, int c);

template <> __device__ __forceinline__ Pair load_pair<float>(const float* row, int c) {
    float2 f = *reinterpret_cast<const float2*>(row + c);
    return {f.x, f.y};
}
template <> __device__ __forceinline__ Pair load_pair<uint16_t>(const uint16_t* row, int c) {
    uint32_t w = *reinterpret_cast<const uint32_t*>(row + c);
    return {bf16_bits_to_f32(w & 0xFFFFu), bf16_bits_to_f32(w >> 16)};
}

struct GroupParams {
    float s, z;
    uint32_t word;     // fp16 s in bits 0..15, fp16 z in bits 16..31
    float h1, h2, h3;  // decision thresholds of code_of: s/2, 3s/2, 5s/2 (infinite when s == 0)
};

// fl32(r / 3) for r >= 0 without the divide sequence: q0 = fl(r c) with
// c = fl32(1/3), then one fma correction step.  Checked exhaustively against the
// IEEE quotient for every finite r >= 0 (bit-identical); r = +inf is taken apart.
__device__ __forceinline__ float div3(float r) {
    const float c = 1.0f / 3.0f;
    const float q0 = r * c;
    const float q1 = fmaf(fmaf(-3.0f, q0, r), c, q0);
    return r <= 0x1.fffffep127f ? q1 : INFINITY;
}

__device__ __forceinline__ GroupParams group_params(float mn, float mx) {
    float rng = mx - mn;
    float s32 = div3(rng);
    uint32_t sb = f32_to_half_bits_rn(s32);
    uint32_t zb = f32_to_half_bits_rn(mn);
    const float s = half_bits_to_f32(sb);
    const bool zero = s == 0.0f;
    return {s, half_bits_to_f32(zb), sb | (zb << 16),
            zero ? INFINITY : 0.5f * s, zero ? INFINITY : 1.5f * s, zero ? INFINITY : 2.5f * s};
}

// code = s == 0 ? 0 : clamp(rint(u), 0, 3) with u = fl32(d / s), d = fl32(x - z), decided
// without dividing.  Round-half-even is monotone, so
//   rint(u) >= 1  <=>  u > 0.5  <=>  d / s > 0.5 + 2^-25   (the rounding midpoint above 0.5 ties to 0.5)
//   rint(u) >= 2  <=>  u >= 1.5 <=>  d / s >= 1.5 - 2^-24  (the midpoint below 1.5 ties to 1.5)
//   rint(u) >= 3  <=>  u > 2.5  <=>  d / s > 2.5 + 2^-23
// With s > 0 an fp16 value (11 significant bits), s/2, 3s/2 and 5s/2 are exact in fp32 and each
// bound s (c + t) lies less than one fp32 ulp from c s, on the side that makes the fp32 decision
// d > s/2, d >= 3s/2, d > 5s/2 (no fp32 value falls between c s and the bound).  Checked for every
// positive fp16 s against the division (tests/test_code_thresholds_exhaustive.py).  With s == 0 the
// thresholds are infinite and the code is 0.  The code is the number of tests passed, so its
// high bit is d >= 3s/2 and its low bit the parity of the three outcomes.  The bits are kept as
// the wave's comparison masks (bit l: lane l), so the parity is two scalar XORs.
struct Code {
    uint64_t hi, lo;
};
__device__ __forceinline__ Code code_of(float x, const GroupParams& p) {
    const float d = x - p.z;
    const uint64_t m1 = __builtin_amdgcn_ballot_w64(d > p.h1);
    const uint64_t m2 = __builtin_amdgcn_ballot_w64(d >= p.h2);
    const uint64_t m3 = __builtin_amdgcn_ballot_w64(d > p.h3);
    return {m2, m1 ^ m2 ^ m3};
}

// Packed codes are built a bit at a time from the most significant end:
// w <- 2 w + (bit of this lane in m), one add whose carry-in is the mask.
// (Written out: the compiler would otherwise select each bit to 0 / 1 and
// shift it into place, three operations per bit.)
__device__ __forceinline__ uint32_t push_bit(uint32_t w, uint64_t m) {
    uint32_t r;
    uint64_t carry_out;
    asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry_out) : "v"(w), "s"(m));
    return r;
}
__device__ __forceinline__ uint32_t push_code(uint32_t w, Code c) { return push_bit(push_bit(w, c.hi), c.lo); }

// Where one call packs: tokens 0..n-1 of its selection (index row stride
// idx_stride) go to tokens tok0.. of a destination laid out for tok_stride
// tokens and grp_stride key groups per (sequence, KV head); tok0 is a multiple
// of 32, so destination groups are whole.
struct PackGeom {
    int n, idx_stride, tok_stride, grp_stride, tok0;
};


// ---- one group of 32 kept rows, loaded whole ----
// A wave reads the group's 32 rows (K or V) as 16-byte chunks, every load
// instruction covering RPI whole rows: lane l takes chunk c = l % CH of rows
// NI r .. NI r + NI - 1, r = l / CH.  Each lane so holds NI rows x EPC
// channels.  Rows are read through a buffer resource over the (sequence, KV
// head) slice: a position outside [0, T) reads as zeros instead of faulting.
template <typename T, int D>
struct Tile {
    static constexpr int EPC = 16 / (int)sizeof(T);  // channels per 16-byte chunk
    static constexpr int CH = D / EPC;                // chunks per row
    static constexpr int RPI = kWave / CH;            // rows per load instruction
    static constexpr int NI = kGroup / RPI;           // rows per lane
    static_assert(CH * RPI == kWave && NI * RPI == kGroup, "tile shape");
};

template <typename T>
__device__ __forceinline__ float elem(const u32x4& x, int e) {  // e: compile-time after unrolling
    if constexpr (std::is_same_v<T, float>) {
        return __uint_as_float(x[e]);
    } else {
        const uint32_t w = x[e / 2];
        return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
}
// The same value, widened by an operation the compiler cannot merge with
// elem(): a pass that reads every element once more later widens again (one
// operation) instead of holding all widened values in registers in between.
template <typename T>
__device__ __forceinline__ float elem_once(const u32x4& x, int e) {
    if constexpr (std::is_same_v<T, float>) {
        return __uint_as_float(x[e]);
    } else {
        const uint32_t w = x[e / 2];
        uint32_t r;
        if (e & 1) asm("v_and_b32 %0, 0xffff0000, %1" : "=v"(r) : "v"(w));
        else asm("v_lshlrev_b32 %0, 16, %1" : "=v"(r) : "v"(w));
        return __uint_as_float(r);
    }
}

// Rows t0 + NI r + q (q < NI) of the call's selection for this lane; tokens at
// or past n read position 0 (their values are never used).
template <typename T, int D>
__device__ __forceinline__ void load_tile(const T* __restrict__ x, const int32_t* __restrict__ idx, int T_ctx,
                                          const PackGeom& pg, int unit, int t0, int lane,
                                          u32x4 (&X)[Tile<T, D>::NI]) {
    using G = Tile<T, D>;
    const int c = lane % G::CH, r = lane / G::CH;
    const auto rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(x + (size_t)unit * T_ctx * D), 0,
                                                      T_ctx * D * (int)sizeof(T), 0x00020000);
    int pos[G::NI];
    if (idx) {  // wave-uniform
        const auto ri = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(idx + (size_t)unit * pg.idx_stride), 0,
                                                          pg.n * 4, 0x00020000);
#pragma unroll
        for (int q = 0; q < G::NI; ++q) pos[q] = (int)__builtin_amdgcn_raw_buffer_load_b32(ri, (t0 + G::NI * r + q) * 4, 0, 0);
    } else {
#pragma unroll
        for (int q = 0; q < G::NI; ++q) pos[q] = t0 + G::NI * r + q;
    }
    // each row is read once: non-temporal loads (cache policy nt) keep them from
    // displacing other data in L2 / MALL
#pragma unroll
    for (int q = 0; q < G::NI; ++q)
        X[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (pos[q] * D + G::EPC * c) * (int)sizeof(T), 0, 2));
}

// ---- combining the lanes that hold other rows of the same chunk ----
// Those lanes differ in lane bits log2(CH) .. 5.  A permlane swap of two
// registers A, B across lane bit 4 (16) or 5 (32) leaves the lanes with that
// bit clear holding (own A, partner's A) and the others (partner's B, own B),
// so one swap and one min / max reduce a pair of entries to one, each lane
// keeping the entry its bit selects (a reduce-scatter); the same swap applied
// to a value and a copy of it hands the entries back (an all-gather).  Bit 3
// (only when CH = 8) is reduced in full by DPP.
template <int B>  // lane bit 4 or 5
__device__ __forceinline__ void swap_pair(float& a, float& b) {
    if constexpr (B == 4) {
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        a = __uint_as_float(p[0]);
        b = __uint_as_float(p[1]);
    } else {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        a = __uint_as_float(p[0]);
        b = __uint_as_float(p[1]);
    }
}
// Entries i and i + N/2 (i < N/2) of mn / mx become entry i: the lanes with
// bit B clear keep entry i's label, the others entry i + N/2's.
template <int B, int N>
__device__ __forceinline__ void scatter_stage(float (&mn)[N], float (&mx)[N]) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
        float a = mn[i], b = mn[i + N / 2];
        swap_pair<B>(a, b);
        mn[i] = fminf(a, b);
        a = mx[i], b = mx[i + N / 2];
        swap_pair<B>(a, b);
        mx[i] = fmaxf(a, b);
    }
}
// The inverse hand-back for one quantity: entries i (i < N) become entries i
// (label with bit B clear) and i + N (bit B set).
template <int B, int N, int M>
__device__ __forceinline__ void gather_stage(float (&v)[M]) {
    static_assert(M >= 2 * N, "room for the handed-back entries");
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float a = v[i], b = v[i];
        swap_pair<B>(a, b);
        v[i] = a;
        v[i + N] = b;
    }
}

// Keys (quantised per channel over the group's cnt tokens).  Each lane folds
// its EPC channels over its NI rows, the lanes of the same chunk combine, and
// every lane derives its channels' parameters.  A token's codes for the
// lane's channels are 2 EPC bits of the token's packed row; they are written
// to the wave's staging area in the packed order and copied out as whole
// 16-byte pieces (only rows below cnt).
template <typename T, int D, bool kFull>
__device__ __forceinline__ void pack_keys_tile(const u32x4 (&X)[Tile<T, D>::NI], int cnt, const PackGeom& pg, int gi,
                                               int unit, int lane, uint8_t* __restrict__ stage,
                                               uint8_t* __restrict__ k_codes, uint32_t* __restrict__ k_sz) {
    using G = Tile<T, D>;
    constexpr int EPC = G::EPC, NI = G::NI;
    const int c = lane % G::CH, r = lane / G::CH;
    float mn[EPC], mx[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
        mn[e] = kFull ? elem_once<T>(X[0], e) : INFINITY;
        mx[e] = kFull ? mn[e] : -INFINITY;
#pragma unroll
        for (int q = kFull ? 1 : 0; q < NI; ++q) {
            const float v = elem_once<T>(X[q], e);
            const bool ok = kFull || NI * r + q < cnt;
            mn[e] = fminf(mn[e], ok ? v : INFINITY);
            mx[e] = fmaxf(mx[e], ok ? v : -INFINITY);
        }
        if constexpr (G::CH <= 8) {  // lane bit 3: row_ror:8
            mn[e] = fminf(mn[e], __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, mn[e]), 0x128, 0xF, 0xF, false)));
            mx[e] = fmaxf(mx[e], __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, mx[e]), 0x128, 0xF, 0xF, false)));
        }
    }
    // Reduce-scatter over lane bits 4 (when CH <= 16) and 5: the lane ends with
    // NE channels, entry i being channel i + (EPC / 4) b5 + (EPC / 2) b4 (both
    // stages) or i + (EPC / 2) b5 (bit 5 only), b4 / b5 its lane bits.
    constexpr bool kB4 = G::CH <= 16;
    constexpr int NE = kB4 ? EPC / 4 : EPC / 2;
    static_assert(NE >= 1, "a lane keeps at least one channel");
    float zz[EPC], h1[EPC], h2[EPC], h3[EPC];
    {
        float m1[EPC / 2], x1[EPC / 2];
        if constexpr (kB4) {
            scatter_stage<4, EPC>(mn, mx);
#pragma unroll
            for (int i = 0; i < EPC / 2; ++i) { m1[i] = mn[i]; x1[i] = mx[i]; }
            scatter_stage<5, EPC / 2>(m1, x1);
        } else {
            scatter_stage<5, EPC>(mn, mx);
#pragma unroll
            for (int i = 0; i < EPC / 2; ++i) { m1[i] = mn[i]; x1[i] = mx[i]; }
        }
        const int b4 = (lane >> 4) & 1, b5 = lane >> 5;
        const int first = kB4 ? (EPC / 4) * b5 + (EPC / 2) * b4 : (EPC / 2) * b5;  // channel of entry 0
        uint32_t words[NE];
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            const GroupParams p = group_params(m1[i], x1[i]);
            words[i] = p.word;
            zz[i] = p.z;
            h1[i] = p.h1;
            h2[i] = p.h2;
            h3[i] = p.h3;
        }
        uint32_t* dst = k_sz + ((size_t)unit * pg.grp_stride + pg.tok0 / kGroup + gi) * D + EPC * c + first;
        if constexpr (NE == 2) *reinterpret_cast<uint2*>(dst) = make_uint2(words[0], words[1]);
        else dst[0] = words[0];
    }
    // All-gather the code thresholds back to every lane of the chunk (bit 5, then bit 4).
    gather_stage<5, NE>(zz);
    gather_stage<5, NE>(h1);
    gather_stage<5, NE>(h2);
    gather_stage<5, NE>(h3);
    if constexpr (kB4) {
        gather_stage<4, 2 * NE>(zz);
        gather_stage<4, 2 * NE>(h1);
        gather_stage<4, 2 * NE>(h2);
        gather_stage<4, 2 * NE>(h3);
    }
    GroupParams pk[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
        pk[e].z = zz[e];
        pk[e].h1 = h1[e];
        pk[e].h2 = h2[e];
        pk[e].h3 = h3[e];
    }
    // token q's codes: channel e in bits 2e .. 2e + 1 of a 2 EPC-bit field
    constexpr int FB = 2 * EPC;
#pragma unroll
    for (int q = 0; q < NI; ++q) {
        uint32_t f = 0u;
#pragma unroll
        for (int e = EPC - 1; e >= 0; --e) f = push_code(f, code_of(elem<T>(X[q], e), pk[e]));
        uint8_t* dst = stage + (NI * r + q) * (D / 4) + c * (FB / 8);
        if constexpr (FB == 16) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)f;
        else *dst = (uint8_t)f;
    }
    constexpr int BYTES = kGroup * D / 4;  // the group's packed rows
    if (16 * lane < BYTES && 16 * lane < cnt * (D / 4)) {
        const uint4 w = *reinterpret_cast<const uint4*>(stage + 16 * lane);
        *reinterpret_cast<uint4*>(k_codes + ((size_t)unit * pg.tok_stride + pg.tok0 + gi * kGroup) * (D / 4) + 16 * lane) = w;
    }
}

// Values (quantised per token over 32-channel groups).  A group is GC = 32 / EPC
// neighbouring lanes of one row; each lane folds its EPC channels per token,
// the GC lanes combine by DPP, and every lane derives its rows' parameters.
// A channel's codes over the lane's rows are 2 NI bits of the channel's 64-bit
// word (token t at bits 2t); they are written to the staging area in the
// packed order (all D channels of the block, tokens past cnt as code 0) and
// copied out as 16-byte pieces, the scale / zero words likewise (rows below cnt).
template <typename T, int D, bool kFull>
__device__ __forceinline__ void pack_values_tile(const u32x4 (&X)[Tile<T, D>::NI], int cnt, const PackGeom& pg,
                                                 int gi, int unit, int lane, uint8_t* __restrict__ stage,
                                                 uint8_t* __restrict__ v_codes, uint32_t* __restrict__ v_sz) {
    using G = Tile<T, D>;
    constexpr int EPC = G::EPC, NI = G::NI, GC = kGroup / EPC, NG = D / kGroup;
    const int c = lane % G::CH, r = lane / G::CH;
    // Rows one at a time: the token's minimum / maximum, parameters and codes;
    // channel e's field f[e] takes token q's code in bits 2q .. 2q + 1 (2 NI-bit
    // fields; rows are pushed from the last, so bits fill from the top).
    constexpr int FB = 2 * NI;
    uint32_t* sz_stage = reinterpret_cast<uint32_t*>(stage + D * 8);
    uint32_t f[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) f[e] = 0u;
#pragma unroll
    for (int q = NI - 1; q >= 0; --q) {
        float mn = elem<T>(X[q], 0), mx = mn;
#pragma unroll
        for (int e = 1; e < EPC; ++e) {
            mn = fminf(mn, elem<T>(X[q], e));
            mx = fmaxf(mx, elem<T>(X[q], e));
        }
        mn = dpp_min<GC>(mn);
        mx = dpp_max<GC>(mx);
        const GroupParams p = group_params(mn, mx);
        if (c % GC == 0) sz_stage[(NI * r + q) * NG + c / GC] = p.word;
        const uint64_t valid = kFull ? ~0ull : __builtin_amdgcn_ballot_w64(NI * r + q < cnt);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
            Code cd = code_of(elem<T>(X[q], e), p);
            cd.hi &= valid;
            cd.lo &= valid;
            f[e] = push_code(f[e], cd);
        }
    }
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
        uint8_t* dst = stage + (EPC * c + e) * 8 + r * (FB / 8);
        if constexpr (FB == 32) *reinterpret_cast<uint32_t*>(dst) = f[e];
        else if constexpr (FB == 16) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)f[e];
        else *dst = (uint8_t)f[e];
    }
    if (16 * lane < D * 8) {
        const uint4 w = *reinterpret_cast<const uint4*>(stage + 16 * lane);
        *reinterpret_cast<uint4*>(v_codes + ((size_t)unit * pg.grp_stride + pg.tok0 / kGroup + gi) * D * 8 + 16 * lane) = w;
    }
    if (lane < cnt) {  // token `lane`'s NG words
        uint32_t* dst = v_sz + ((size_t)unit * pg.tok_stride + pg.tok0 + gi * kGroup + lane) * NG;
        if constexpr (NG == 4) *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(sz_stage + lane * NG);
        else *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(sz_stage + lane * NG);
    }
}

// Bytes of one wave's staging area: packed codes of a group (8 D) and, for
// values, its scale / zero words (4 D).
template <int D>
constexpr int kStageBytes = 12 * D;

// One workgroup per (group of 32 kept tokens, KV head, sequence): wave 0 packs
// the keys, wave 1 the values.
template <typename T, int D>
__global__ __launch_bounds__(128) void quant_pack_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ idx, int T_ctx, PackGeom pg,
    int Hkv, uint8_t* __restrict__ k_codes, uint32_t* __restrict__ k_sz, uint8_t* __restrict__ v_codes,
    uint32_t* __restrict__ v_sz) {
    __shared__ __align__(16) uint8_t stage[2][kStageBytes<D>];
    const int gi = blockIdx.x;
    const int cnt = min(kGroup, pg.n - gi * kGroup);
    const int unit = blockIdx.z * Hkv + blockIdx.y;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    u32x4 X[Tile<T, D>::NI];
    load_tile<T, D>(wave == 0 ? k : v, idx, T_ctx, pg, unit, gi * kGroup, lane, X);
    // full groups (all but a call's last) take the branch-free instance
    if (wave == 0) {
        if (cnt == kGroup) pack_keys_tile<T, D, true>(X, cnt, pg, gi, unit, lane, stage[0], k_codes, k_sz);
        else pack_keys_tile<T, D, false>(X, cnt, pg, gi, unit, lane, stage[0], k_codes, k_sz);
    } else {
        if (cnt == kGroup) pack_values_tile<T, D, true>(X, cnt, pg, gi, unit, lane, stage[1], v_codes, v_sz);
        else pack_values_tile<T, D, false>(X, cnt, pg, gi, unit, lane, stage[1], v_codes, v_sz);
    }
}

// One generation step's append with the counts in device memory
// (counts = {n_packed, n_res, overflow, ticket}): workgroup (g, b) of grid
// (1, Hkv, B) copies the new K row (wave 0) and V row (wave 1) into window slot
// n_res; when that slot was the window's last, the same waves pack the window
// as group n_packed / 32 (the rule of quant_pack_kernel) or, with no capacity
// left, the overflow flag is raised.  Every workgroup reads the counts before
// it takes a ticket, so the workgroup that takes the last ticket can advance
// them: no other launch, no spinning.  The ticket needs no memory fence: each
// workgroup's reads of the counts have returned before its barrier (every
// thread's stores depend on them), and what the step writes (rows, packed
// group, counts) is read by later launches, which the kernel boundary orders.
// (A device-scope fence here writes back and invalidates the L2 of the
// workgroup's XCD.)
template <int D>
__global__ __launch_bounds__(128) void stream_step_append_kernel(
    const uint32_t* __restrict__ k_new, const uint32_t* __restrict__ v_new, int Hkv, int cap,
    int32_t* __restrict__ counts, uint16_t* __restrict__ k_res, uint16_t* __restrict__ v_res,
    uint8_t* __restrict__ k_codes, uint32_t* __restrict__ k_sz, uint8_t* __restrict__ v_codes,
    uint32_t* __restrict__ v_sz) {
    constexpr int W = D / 2;  // dwords per bf16 row
    __shared__ __align__(16) uint8_t stage[2][kStageBytes<D>];
    const int unit = blockIdx.z * Hkv + blockIdx.y;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int n_packed = counts[0], n_res = counts[1], flag = counts[2];
    const bool ok = flag == 0 && n_res >= 0 && n_res < kGroup && n_packed >= 0 && n_packed % kGroup == 0 &&
                    n_packed <= cap;
    const bool full = ok && n_res == kGroup - 1;
    const bool pack = full && n_packed + kGroup <= cap;
    if (ok && lane < W) {
        const uint32_t* src = (wave == 0 ? k_new : v_new) + (size_t)unit * W;
        uint32_t* dst = reinterpret_cast<uint32_t*>(wave == 0 ? k_res : v_res) + ((size_t)unit * kGroup + n_res) * W;
        dst[lane] = src[lane];
    }
    __syncthreads();  // the new row is visible to both waves
    if (pack) {
        const PackGeom pg{kGroup, kGroup, cap, cap / kGroup, n_packed};
        u32x4 X[Tile<uint16_t, D>::NI];
        load_tile<uint16_t, D>(wave == 0 ? k_res : v_res, nullptr, kGroup, pg, unit, 0, lane, X);
        if (wave == 0) pack_keys_tile<uint16_t, D, true>(X, kGroup, pg, 0, unit, lane, stage[0], k_codes, k_sz);
        else pack_values_tile<uint16_t, D, true>(X, kGroup, pg, 0, unit, lane, stage[1], v_codes, v_sz);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int nwg = (int)(gridDim.y * gridDim.z);
        if (atomicAdd(&counts[3], 1) == nwg - 1) {  // every workgroup has read the counts
            if (ok) {
                if (!full) {
                    counts[1] = n_res + 1;
                } else if (pack) {
                    counts[0] = n_packed + kGroup;
                    counts[1] = 0;
                } else {
                    counts[2] = 1;
                }
            }
            counts[3] = 0;
        }
    }
}

template <typename T, int D>
hipError_t launch_typed(const void* k, const void* v, const int32_t* idx, int B, int Hkv, int T_ctx,
                        const PackGeom& pg, uint8_t* k_codes, uint32_t* k_sz, uint8_t* v_codes, uint32_t* v_sz,
                        hipStream_t stream) {
    const int G = (pg.n + kGroup - 1) / kGroup;
    hipLaunchKernelGGL((quant_pack_kernel<T, D>), dim3(G, Hkv, B), dim3(128), 0, stream, static_cast<const T*>(k),
                       static_cast<const T*>(v), idx, T_ctx, pg, Hkv, k_codes, k_sz, v_codes, v_sz);
    return hipGetLastError();
}

hipError_t launch_geom(const void* k, const void* v, bool bf16, const int32_t* idx, int B, int Hkv, int T_ctx,
                       int D, const PackGeom& pg, uint8_t* k_codes, uint32_t* k_sz, uint8_t* v_codes,
                       uint32_t* v_sz, hipStream_t stream) {
    if (bf16) {
        if (D == 128) return launch_typed<uint16_t, 128>(k, v, idx, B, Hkv, T_ctx, pg, k_codes, k_sz, v_codes, v_sz, stream);
        return launch_typed<uint16_t, 64>(k, v, idx, B, Hkv, T_ctx, pg, k_codes, k_sz, v_codes, v_sz, stream);
    }
    if (D == 128) return launch_typed<float, 128>(k, v, idx, B, Hkv, T_ctx, pg, k_codes, k_sz, v_codes, v_sz, stream);
    return launch_typed<float, 64>(k, v, idx, B, Hkv, T_ctx, pg, k_codes, k_sz, v_codes, v_sz, stream);
}

}  // namespace

hipError_t launch_quant_pack(const void* k, const void* v, bool bf16, const int32_t* idx, int B,
                             int Hkv, int T_ctx, int D, int n_keep, uint8_t* k_codes, uint32_t* k_sz,
                             uint8_t* v_codes, uint32_t* v_sz, hipStream_t stream) {
    const PackGeom pg{n_keep, n_keep, n_keep, (n_keep + kGroup - 1) / kGroup, 0};
    return launch_geom(k, v, bf16, idx, B, Hkv, T_ctx, D, pg, k_codes, k_sz, v_codes, v_sz, stream);
}

hipError_t launch_stream_step_append(const void* k_new, const void* v_new, int B, int Hkv, int D, int cap,
                                     int32_t* counts, uint8_t* k_codes, uint32_t* k_sz, uint8_t* v_codes,
                                     uint32_t* v_sz, void* k_res, void* v_res, hipStream_t stream) {
    const dim3 grid(1, Hkv, B);
    if (D == 128)
        hipLaunchKernelGGL((stream_step_append_kernel<128>), grid, dim3(128), 0, stream,
                           static_cast<const uint32_t*>(k_new), static_cast<const uint32_t*>(v_new), Hkv, cap, counts,
                           static_cast<uint16_t*>(k_res), static_cast<uint16_t*>(v_res), k_codes, k_sz, v_codes, v_sz);
    else
        hipLaunchKernelGGL((stream_step_append_kernel<64>), grid, dim3(128), 0, stream,
                           static_cast<const uint32_t*>(k_new), static_cast<const uint32_t*>(v_new), Hkv, cap, counts,
                           static_cast<uint16_t*>(k_res), static_cast<uint16_t*>(v_res), k_codes, k_sz, v_codes, v_sz);
    return hipGetLastError();
}

hipError_t launch_stream_pack(const void* k, const void* v, bool bf16, const int32_t* idx, int idx_stride, int B,
                              int Hkv, int T_ctx, int D, int n, int cap, int tok0, uint8_t* k_codes,
                              uint32_t* k_sz, uint8_t* v_codes, uint32_t* v_sz, hipStream_t stream) {
    const PackGeom pg{n, idx_stride, cap, cap / kGroup, tok0};
    return launch_geom(k, v, bf16, idx, B, Hkv, T_ctx, D, pg, k_codes, k_sz, v_codes, v_sz, stream);
}

}  // namespace minikv
