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
// tests (code_of: three comparisons with exact multiples of s) and match a
// plain IEEE evaluation of the rule bit for bit.
// Inputs are finite (-fno-honor-nans: min / max need no NaN handling).
//
// HBM-bound gather: each kept row is read once (coalesced 4-byte lane loads of
// two channels), each packed byte written once (key codes: dword stores
// assembled with DPP ORs; value codes: one 16-byte store per lane).  Keys and
// values of a token group are packed by the two waves of one workgroup.
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
// thresholds are infinite and the code is 0.  The three tests are taken as a two-step search:
// d >= 3s/2 decides the high bit, and the low bit is d > 5s/2 above it or d > s/2 below it (the
// same decisions, one comparison fewer).
__device__ __forceinline__ uint32_t code_of(float x, const GroupParams& p) {
    const float d = x - p.z;
    const bool hi = d >= p.h2;
    return (hi ? 2u : 0u) + (uint32_t)(d > (hi ? p.h3 : p.h1));
}

// Where one call packs: tokens 0..n-1 of its selection (index row stride
// idx_stride) go to tokens tok0.. of a destination laid out for tok_stride
// tokens and grp_stride key groups per (sequence, KV head); tok0 is a multiple
// of 32, so destination groups are whole.
struct PackGeom {
    int n, idx_stride, tok_stride, grp_stride, tok0;
};

// Lane S of each 16-lane row, to the whole row (DPP row_newbcast).
template <int S>
__device__ __forceinline__ float row_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + S, 0xF, 0xF, false));
}

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// One stage of the row reduce-scatter: lanes paired by DPP pattern P (which
// flips bit B of lane % 16, among others already resolved) exchange the
// tokens whose bit B differs from their own and keep the min / max of the
// rest; slot t (bit B of t clear) ends with the kept token's value.
template <int P, int B>
__device__ __forceinline__ void rs_stage(float (&mn)[kGroup], float (&mx)[kGroup], int lane) {
    const bool hi = (lane >> B) & 1;
    static_for<0, kGroup>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        if constexpr ((t & (1 << B)) == 0) {
            constexpr int u = t | (1 << B);
            const float kmn = hi ? mn[u] : mn[t], smn = hi ? mn[t] : mn[u];
            const float kmx = hi ? mx[u] : mx[t], smx = hi ? mx[t] : mx[u];
            mn[t] = fminf(kmn, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, smn), P, 0xF, 0xF, false)));
            mx[t] = fmaxf(kmx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, smx), P, 0xF, 0xF, false)));
        }
    });
}

// Per-token min / max over each 16-lane row, scattered: afterwards mn[0],
// mx[0] hold token lane % 16 and mn[16], mx[16] token 16 + lane % 16.  The
// partners are row_mirror (lane ^ 15), row_half_mirror (^ 7), quad_perm
// [3,2,1,0] (^ 3) and [1,0,3,2] (^ 1); each flips the bit it resolves and, besides
// it, only bits still unresolved, so partners always hold the same tokens.
__device__ __forceinline__ void row_reduce_scatter(float (&mn)[kGroup], float (&mx)[kGroup], int lane) {
    rs_stage<0x140, 3>(mn, mx, lane);
    rs_stage<0x141, 2>(mn, mx, lane);
    rs_stage<0x1B, 1>(mn, mx, lane);
    rs_stage<0xB1, 0>(mn, mx, lane);
}

// OR over aligned groups of 8 lanes: quad swaps, then the mirrored half row.
__device__ __forceinline__ uint32_t or8(uint32_t x) {
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, true);  // row_half_mirror
    return x;
}

// Keys: one wave per (group of 32 kept tokens, KV head, sequence).
// Lane l owns channels 2l, 2l+1 (D/2 active lanes).
template <typename T, int D>
__device__ __forceinline__ void pack_keys(
    const T* __restrict__ k, const int32_t* __restrict__ idx, int T_ctx, const PackGeom& pg, int gi, int unit,
    uint8_t* __restrict__ k_codes, uint32_t* __restrict__ k_sz) {
    const int lane = threadIdx.x % kWave;
    const bool active = lane < D / 2;
    const int c = 2 * (active ? lane : 0);
    const int t0 = gi * kGroup;
    const int cnt = min(kGroup, pg.n - t0);
    const T* base = k + (size_t)unit * T_ctx * D;
    const int32_t* ids = idx ? idx + (size_t)unit * pg.idx_stride + t0 : nullptr;

    Pair x[kGroup];
    float mn0 = INFINITY, mx0 = -INFINITY, mn1 = INFINITY, mx1 = -INFINITY;
#pragma unroll
    for (int t = 0; t < kGroup; ++t) {
        if (t < cnt) {
            const int pos = ids ? ids[t] : t0 + t;
            x[t] = load_pair<T>(base + (size_t)pos * D, c);
            mn0 = fminf(mn0, x[t].a); mx0 = fmaxf(mx0, x[t].a);
            mn1 = fminf(mn1, x[t].b); mx1 = fmaxf(mx1, x[t].b);
        } else {
            x[t] = {0.0f, 0.0f};
        }
    }
    const GroupParams p0 = group_params(mn0, mx0);
    const GroupParams p1 = group_params(mn1, mx1);
    if (active) {
        uint2 w = make_uint2(p0.word, p1.word);
        *reinterpret_cast<uint2*>(k_sz + ((size_t)unit * pg.grp_stride + pg.tok0 / kGroup + gi) * D + c) = w;
    }
    uint8_t* crow = k_codes + ((size_t)unit * pg.tok_stride + pg.tok0 + t0) * (D / 4);
#pragma unroll
    for (int t = 0; t < kGroup; ++t) {
        if (t < cnt) {  // uniform across the wave
            uint32_t nib = active ? (code_of(x[t].a, p0) | (code_of(x[t].b, p1) << 2)) : 0u;
            uint32_t word = or8(nib << (4 * (lane & 7)));
            if (active && (lane & 7) == 0)
                *reinterpret_cast<uint32_t*>(crow + (size_t)t * (D / 4) + 4 * (lane >> 3)) = word;
        }
    }
}

// Values: one wave per (block of 32 kept tokens, KV head, sequence).  Lane l
// owns channels 2l, 2l+1 (D/2 active lanes); a 16-lane row is one 32-channel
// group, so each token's min / max is a row reduction.  The codes are gathered
// along tokens: the lane ends with the 32 codes of each of its two channels
// (8 bytes each, the block's token 4m+j in bits 2j..2j+1 of byte m) and stores
// both in one 16-byte write; tokens past the call's count stay code 0.
template <typename T, int D>
__device__ __forceinline__ void pack_values(
    const T* __restrict__ v, const int32_t* __restrict__ idx, int T_ctx, const PackGeom& pg, int gi, int unit,
    uint8_t* __restrict__ v_codes, uint32_t* __restrict__ v_sz) {
    const int lane = threadIdx.x % kWave;
    const bool active = lane < D / 2;
    const int c = 2 * (active ? lane : 0);
    const int t0 = gi * kGroup;
    const int cnt = min(kGroup, pg.n - t0);
    const T* base = v + (size_t)unit * T_ctx * D;
    const int32_t* ids = idx ? idx + (size_t)unit * pg.idx_stride + t0 : nullptr;

    Pair x[kGroup];
#pragma unroll
    for (int t = 0; t < kGroup; ++t) {
        x[t] = {0.0f, 0.0f};
        if (t < cnt && active) {
            const int pos = ids ? ids[t] : t0 + t;
            x[t] = load_pair<T>(base + (size_t)pos * D, c);
        }
    }
    uint32_t wa[2] = {0u, 0u}, wb[2] = {0u, 0u};
#pragma unroll
    for (int t = 0; t < kGroup; ++t) {
        if (t < cnt) {  // uniform across the wave
            const float mn = dpp_min<16>(fminf(x[t].a, x[t].b));
            const float mx = dpp_max<16>(fmaxf(x[t].a, x[t].b));
            const GroupParams p = group_params(mn, mx);
            wa[t / 16] |= code_of(x[t].a, p) << (2 * (t % 16));
            wb[t / 16] |= code_of(x[t].b, p) << (2 * (t % 16));
            if (active && (lane & 15) == 0)
                v_sz[((size_t)unit * pg.tok_stride + pg.tok0 + t0 + t) * (D / 32) + (lane >> 4)] = p.word;
        }
    }
    if (active)
        *reinterpret_cast<uint4*>(v_codes + (((size_t)unit * pg.grp_stride + pg.tok0 / kGroup + gi) * D + c) * 8) =
            make_uint4(wa[0], wa[1], wb[0], wb[1]);
}

// Full groups (32 kept tokens): the same rule without per-token branches.  Rows
// are gathered through a buffer resource sized to the head's T rows (a position
// outside [0, T) reads as zeros instead of faulting); key-code words and value
// parameters are collected in registers and written four and two stores per
// lane at the end.
template <typename T> __device__ __forceinline__ Pair load_pair_buf(__amdgpu_buffer_rsrc_t r, int off);
template <> __device__ __forceinline__ Pair load_pair_buf<float>(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    return {__uint_as_float(w.x), __uint_as_float(w.y)};
}
template <> __device__ __forceinline__ Pair load_pair_buf<uint16_t>(__amdgpu_buffer_rsrc_t r, int off) {
    const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    return {bf16_bits_to_f32(w & 0xFFFFu), bf16_bits_to_f32(w >> 16)};
}

template <typename T, int D>
__device__ __forceinline__ void gather_full(const T* __restrict__ x, const int32_t* __restrict__ idx, int T_ctx,
                                            int idx_stride, int unit, int t0, int c, Pair (&out)[kGroup]) {
    const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(x + (size_t)unit * T_ctx * D), 0,
                                                     T_ctx * D * (int)sizeof(T), 0x00020000);
    if (idx) {  // one branch per wave: the positions are read once, as scalars
        const int32_t* ids = idx + (size_t)unit * idx_stride + t0;
        int pos[kGroup];
#pragma unroll
        for (int t = 0; t < kGroup; ++t) pos[t] = ids[t];
#pragma unroll
        for (int t = 0; t < kGroup; ++t) out[t] = load_pair_buf<T>(r, (pos[t] * D + c) * (int)sizeof(T));
    } else {
#pragma unroll
        for (int t = 0; t < kGroup; ++t) out[t] = load_pair_buf<T>(r, ((t0 + t) * D + c) * (int)sizeof(T));
    }
}

template <typename T, int D>
__device__ __forceinline__ void pack_keys_full(
    const T* __restrict__ k, const int32_t* __restrict__ idx, int T_ctx, const PackGeom& pg, int gi, int unit,
    uint8_t* __restrict__ k_codes, uint32_t* __restrict__ k_sz) {
    const int lane = threadIdx.x % kWave;
    const bool active = lane < D / 2;
    const int c = 2 * (active ? lane : 0);
    const int t0 = gi * kGroup;
    Pair x[kGroup];
    gather_full<T, D>(k, idx, T_ctx, pg.idx_stride, unit, t0, c, x);
    float mn0 = x[0].a, mx0 = x[0].a, mn1 = x[0].b, mx1 = x[0].b;
#pragma unroll
    for (int t = 1; t < kGroup; ++t) {
        mn0 = fminf(mn0, x[t].a); mx0 = fmaxf(mx0, x[t].a);
        mn1 = fminf(mn1, x[t].b); mx1 = fmaxf(mx1, x[t].b);
    }
    const GroupParams p0 = group_params(mn0, mx0);
    const GroupParams p1 = group_params(mn1, mx1);
    if (active) *reinterpret_cast<uint2*>(k_sz + ((size_t)unit * pg.grp_stride + pg.tok0 / kGroup + gi) * D + c) = make_uint2(p0.word, p1.word);
    // Token t's word for channel block lane / 8 is kept by the lane with lane % 8 == t % 8.
    uint32_t kw[kGroup / 8] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < kGroup; ++t) {
        const uint32_t nib = code_of(x[t].a, p0) | (code_of(x[t].b, p1) << 2);
        const uint32_t word = or8(nib << (4 * (lane & 7)));
        kw[t / 8] = (lane & 7) == (t & 7) ? word : kw[t / 8];
    }
    uint8_t* crow = k_codes + ((size_t)unit * pg.tok_stride + pg.tok0 + t0) * (D / 4);
    if (active) {
#pragma unroll
        for (int m = 0; m < kGroup / 8; ++m)
            *reinterpret_cast<uint32_t*>(crow + (size_t)(8 * m + (lane & 7)) * (D / 4) + 4 * (lane >> 3)) = kw[m];
    }
}

template <typename T, int D>
__device__ __forceinline__ void pack_values_full(
    const T* __restrict__ v, const int32_t* __restrict__ idx, int T_ctx, const PackGeom& pg, int gi, int unit,
    uint8_t* __restrict__ v_codes, uint32_t* __restrict__ v_sz) {
    const int lane = threadIdx.x % kWave;
    const bool active = lane < D / 2;
    const int c = 2 * (active ? lane : 0);
    const int t0 = gi * kGroup;
    Pair x[kGroup];
    gather_full<T, D>(v, idx, T_ctx, pg.idx_stride, unit, t0, c, x);
    // Every 16-lane row (32 channels) reduces each token's min / max so that
    // the lane with lane % 16 == j ends with those of tokens j and j + 16
    // (a reduce-scatter), derives their parameters once, and the row reads them
    // back by DPP broadcast, instead of all 16 lanes deriving every token's.
    float mn[kGroup], mx[kGroup];
#pragma unroll
    for (int t = 0; t < kGroup; ++t) {
        mn[t] = fminf(x[t].a, x[t].b);
        mx[t] = fmaxf(x[t].a, x[t].b);
    }
    row_reduce_scatter(mn, mx, lane);
    const float own_mn[2] = {mn[0], mn[16]}, own_mx[2] = {mx[0], mx[16]};
    const GroupParams own[2] = {group_params(own_mn[0], own_mx[0]), group_params(own_mn[1], own_mx[1])};
    uint32_t wa[2] = {0u, 0u}, wb[2] = {0u, 0u};
    const uint32_t vw[2] = {own[0].word, own[1].word};  // token 16 h + lane % 16 of row lane / 16
    static_for<0, kGroup>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        GroupParams p;
        p.z = row_bcast<t & 15>(own[t / 16].z);
        p.h1 = row_bcast<t & 15>(own[t / 16].h1);
        p.h2 = row_bcast<t & 15>(own[t / 16].h2);
        p.h3 = row_bcast<t & 15>(own[t / 16].h3);
        wa[t / 16] |= code_of(x[t].a, p) << (2 * (t % 16));
        wb[t / 16] |= code_of(x[t].b, p) << (2 * (t % 16));
    });
    if (active) {
        *reinterpret_cast<uint4*>(v_codes + (((size_t)unit * pg.grp_stride + pg.tok0 / kGroup + gi) * D + c) * 8) = make_uint4(wa[0], wa[1], wb[0], wb[1]);
#pragma unroll
        for (int h = 0; h < 2; ++h)
            v_sz[((size_t)unit * pg.tok_stride + pg.tok0 + t0 + 16 * h + (lane & 15)) * (D / 32) + (lane >> 4)] = vw[h];
    }
}

// One workgroup per (group of 32 kept tokens, KV head, sequence): wave 0 packs
// the keys, wave 1 the values.
template <typename T, int D>
__global__ __launch_bounds__(128) void quant_pack_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ idx, int T_ctx, PackGeom pg,
    int Hkv, uint8_t* __restrict__ k_codes, uint32_t* __restrict__ k_sz, uint8_t* __restrict__ v_codes,
    uint32_t* __restrict__ v_sz) {
    const bool full = (blockIdx.x + 1) * kGroup <= pg.n;
    const int gi = blockIdx.x;
    const int unit = blockIdx.z * Hkv + blockIdx.y;
    if (threadIdx.x < kWave) {
        if (full) pack_keys_full<T, D>(k, idx, T_ctx, pg, gi, unit, k_codes, k_sz);
        else pack_keys<T, D>(k, idx, T_ctx, pg, gi, unit, k_codes, k_sz);
    } else {
        if (full) pack_values_full<T, D>(v, idx, T_ctx, pg, gi, unit, v_codes, v_sz);
        else pack_values<T, D>(v, idx, T_ctx, pg, gi, unit, v_codes, v_sz);
    }
}

// One generation step's append with the counts in device memory
// (counts = {n_packed, n_res, overflow, ticket}): workgroup (g, b) of grid
// (1, Hkv, B) copies the new K row (wave 0) and V row (wave 1) into window slot
// n_res; when that slot was the window's last, the same waves pack the window
// as group n_packed / 32 (the rule of quant_pack_kernel) or, with no capacity
// left, the overflow flag is raised.  Every workgroup reads the counts before
// it takes a ticket, so the workgroup that takes the last ticket can advance
// them: no other launch, no spinning.
template <int D>
__global__ __launch_bounds__(128) void stream_step_append_kernel(
    const uint32_t* __restrict__ k_new, const uint32_t* __restrict__ v_new, int Hkv, int cap,
    int32_t* __restrict__ counts, uint16_t* __restrict__ k_res, uint16_t* __restrict__ v_res,
    uint8_t* __restrict__ k_codes, uint32_t* __restrict__ k_sz, uint8_t* __restrict__ v_codes,
    uint32_t* __restrict__ v_sz) {
    constexpr int W = D / 2;  // dwords per bf16 row
    const int unit = blockIdx.z * Hkv + blockIdx.y;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
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
        if (wave == 0) pack_keys_full<uint16_t, D>(k_res, nullptr, kGroup, pg, 0, unit, k_codes, k_sz);
        else pack_values_full<uint16_t, D>(v_res, nullptr, kGroup, pg, 0, unit, v_codes, v_sz);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
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
            __threadfence();
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
