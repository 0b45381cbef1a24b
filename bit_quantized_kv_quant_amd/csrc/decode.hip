// Single-query decode attention over the packed 2-bit cache.
//
// Method: paper-listing abstract (the 2-bit layer-discriminative cache serves
// inference) and the gptget.net summary, 方法详解 (per-channel keys, per-token
// values, compact layout).  For query head h on KV head g = h / R:
//   out = sum_t softmax_t(q . khat_t * scale) vhat_t,   xhat = code * s + z
// over the n_keep packed tokens.
//
// HBM-bound: the packed bytes of every kept token are read exactly once; the R
// query heads of a KV head share each read.  Both contractions run on the
// matrix cores so that the vector ALUs only unpack and bookkeep:
//   * a 2-bit code zero-extended to a nibble is the e2m1 (fp4) number code / 2,
//     so `w & 0x33333333` and `(w >> 2) & 0x33333333` turn a 16-code word into
//     an MFMA operand;
//   * the other operand is an fp32 quantity split into e4m3 (fp8) pieces:
//     x = p0 + p1/16 + p2/256 (+ p3/4096), each piece the fp8 rounding of 16^k
//     times what is left, so three (four) pieces carry 12 (16) significant
//     bits of every element and every product with a code is exact; the MFMA
//     rows hold (head, piece), the row's E8M0 scale restores 16^-k, and the
//     pieces are summed after the product, in fp32.
// Keys (16x16x128 f8f6f4, K = channels): per 32-token block the scales fold
// into the query, x_c = q_c s_c (log2 units), scaled by one power of two so
// |x| < 256, split into four pieces and staged through LDS in MFMA K order;
// the zero-point term sum_c q_c z_c is a per-block constant.  One MFMA gives
// 16 tokens' scores for all R heads.
// Values (16x16x128 f8f6f4, K = tokens): values are stored packed along
// tokens (a channel's 32 codes of a block in 8 bytes), the weights w = p s of
// the step's 128 tokens are split into three pieces per (head, value group),
// and one MFMA accumulates 16 channels over 128 tokens; sum_t p z is kept per
// value group on the side.  Softmax runs in the log2 domain, online per
// 128-token step.
//
// Work split: an item is a (sequence, KV head, token range of `chunk`
// tokens, a multiple of 128); enough ranges per KV head to give >= 4096 items.
// The grid holds as many 4-wave workgroups as stay resident, and every wave
// walks its own items (no workgroup barrier): all 128-token steps of an item in
// order, the next step's key loads issued once the current keys are consumed
// and its value loads once the current values are, across item boundaries too.
// With one range per KV head the wave writes the bf16 output itself.  When a
// KV head's ranges fit a few workgroups (small batches) the merge happens in
// the same launch: the workgroups of a head combine their waves' parts in LDS
// and the last one to take the head's ticket merges the workgroups' parts
// (decode_partial_kernel with kTicket), a streaming cache's residual window
// included.  Otherwise partial (m, l, acc) per range go to the workspace and a
// small second kernel merges them (with the window, if any).
#include <algorithm>
#include <atomic>

#include "common.h"
#include "kernels.h"

namespace minikv {
namespace {

constexpr int kStep = 128;        // tokens per wave step: four 32-token blocks
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kScaleOne = 0x7F7F7F7F;  // E8M0 block scale 2^0 for both MFMA operands

// C = A B with A e4m3 (rows x 128 K), B e2m1 (128 K x 16 columns), fp32
// accumulate; sa is this lane's A row scale (E8M0 in every byte).
__device__ __forceinline__ f32x4 mfma_f8_f4(const i32x8& a, const i32x8& b, int sa) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 4, 0, sa, 0,
                                                            kScaleOne);
}

// B operand from 32 codes (two 16-code words): nibble 8d + i of the operand is
// code 2i + (d % 2) of word d / 2, as e2m1 = code / 2.
__device__ __forceinline__ i32x8 codes_e2m1(uint2 w) {
    return i32x8{(int)(w.x & 0x33333333u), (int)((w.x >> 2) & 0x33333333u),
                 (int)(w.y & 0x33333333u), (int)((w.y >> 2) & 0x33333333u), 0, 0, 0, 0};
}

// A operand: 16 bytes at K 16 blk .. and 16 bytes at K 64 + 16 blk .. of a 128-byte row.
__device__ __forceinline__ i32x8 a_operand(const uint8_t* row16) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(row16);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(row16 + 64);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// e4m3 pieces of two values (|x| < 256): x = sum_k 16^-k fp8_k, fp8_k the e4m3
// rounding of 16^k times what the earlier pieces leave, so each piece adds four
// significant bits relative to x itself; piece k of (x0, x1) goes to bytes
// 2(k%2), 2(k%2) + 1 of w[k/2], and P = 3 leaves piece 3 zero.  The 16^-k comes
// back as the E8M0 scale 127 - 4k of the piece's MFMA row.
typedef short s16x2 __attribute__((ext_vector_type(2)));
template <bool kHi>
__device__ __forceinline__ uint32_t fp8_pk(float a, float b, uint32_t old, float scale) {  // fp8(a / scale), fp8(b / scale)
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(s16x2, old), a, b,
                                                                                scale, kHi));
}
__device__ __forceinline__ float pow2_bits(uint32_t biased) { return __builtin_bit_cast(float, biased << 23); }

// e4m3 pieces of x0, x1 relative to the power of two u = 2^(e - 127) (|x| < 256 u):
// x = u sum_k 16^-k fp8_k, fp8_k the e4m3 rounding of 16^k / u times what the
// earlier pieces leave, so each piece adds four significant bits relative to x
// itself.  Piece k of (x0, x1) goes to bytes 2(k%2), 2(k%2) + 1 of w[k/2]; P = 3
// leaves the upper half of w[1] undefined.  The 16^-k comes back as the E8M0
// scale 127 - 4k of the piece's MFMA row, the u as a multiplier after it.
template <int P>
__device__ __forceinline__ void e4m3_pieces(float x0, float x1, uint32_t e, uint32_t (&w)[2]) {
    const float u0 = pow2_bits(e), u1 = pow2_bits(e - 4), u2 = pow2_bits(e - 8), u3 = pow2_bits(e - 12);
    w[0] = fp8_pk<false>(x0, x1, __builtin_nondeterministic_value(0u), u0);
    f32x2 f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[0], u0, false);
    x0 -= f[0];
    x1 -= f[1];
    w[0] = fp8_pk<true>(x0, x1, w[0], u1);
    f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[0], u1, true);
    x0 -= f[0];
    x1 -= f[1];
    w[1] = fp8_pk<false>(x0, x1, __builtin_nondeterministic_value(0u), u2);
    if constexpr (P == 4) {
        f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[1], u2, false);
        x0 -= f[0];
        x1 -= f[1];
        w[1] = fp8_pk<true>(x0, x1, w[1], u3);
    }
}
// Biased exponent of u for a non-negative maximum m (bits): m < 2^8 u, clamped
// so that u 16^-3 stays a normal number (tiny maxima only lose their tail).
__device__ __forceinline__ uint32_t piece_exp(uint32_t m_bits) {
    const int e = (int)(m_bits >> 23) - 7;
    return (uint32_t)(e < 27 ? 27 : e);
}

// Row (16-lane) reductions; each DPP pattern reads inside the row, so the
// shuffle folds into the combining instruction.
template <int kCtrl>
__device__ __forceinline__ uint32_t dppu(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kCtrl, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t row_umax(uint32_t x) {  // non-negative floats as bits
    x = max(x, dppu<0xB1>(x));
    x = max(x, dppu<0x4E>(x));
    x = max(x, dppu<0x141>(x));
    return max(x, dppu<0x140>(x));
}
__device__ __forceinline__ int row_imax(int x) {
    x = max(x, (int)dppu<0xB1>((uint32_t)x));
    x = max(x, (int)dppu<0x4E>((uint32_t)x));
    x = max(x, (int)dppu<0x141>((uint32_t)x));
    return max(x, (int)dppu<0x140>((uint32_t)x));
}
__device__ __forceinline__ float row_fsum(float x) {
    x += __builtin_bit_cast(float, dppu<0xB1>(__builtin_bit_cast(uint32_t, x)));
    x += __builtin_bit_cast(float, dppu<0x4E>(__builtin_bit_cast(uint32_t, x)));
    x += __builtin_bit_cast(float, dppu<0x141>(__builtin_bit_cast(uint32_t, x)));
    return x + __builtin_bit_cast(float, dppu<0x140>(__builtin_bit_cast(uint32_t, x)));
}
// Order-preserving int key of a float (max of keys = key of the max).
__device__ __forceinline__ int fkey(float x) {
    const int b = __builtin_bit_cast(int, x);
    return b ^ (int)((uint32_t)(b >> 31) >> 1);
}
__device__ __forceinline__ float fkey_inv(int k) { return __builtin_bit_cast(float, k ^ (int)((uint32_t)(k >> 31) >> 1)); }

// Four values per lane -> the combination of value r over all 64 lanes, in row r.
// Two permlane32 swaps pair lanes l, l^32 (lower half keeps v0 / v1, upper v2 / v3),
// one permlane16 swap pairs rows (keeping one value per row), DPP finishes the row.
__device__ __forceinline__ uint32_t umax4_rows(uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3) {
    const auto a = __builtin_amdgcn_permlane32_swap(v0, v2, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(v1, v3, false, false);
    const uint32_t t = max(a[0], a[1]), u = max(b[0], b[1]);
    const auto c = __builtin_amdgcn_permlane16_swap(t, u, false, false);
    return row_umax(max(c[0], c[1]));
}
__device__ __forceinline__ float fsum4_rows(float v0, float v1, float v2, float v3) {
    auto bits = [](float x) { return __builtin_bit_cast(uint32_t, x); };
    auto flt = [](uint32_t x) { return __builtin_bit_cast(float, x); };
    const auto a = __builtin_amdgcn_permlane32_swap(bits(v0), bits(v2), false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(bits(v1), bits(v3), false, false);
    const float t = flt(a[0]) + flt(a[1]), u = flt(b[0]) + flt(b[1]);
    const auto c = __builtin_amdgcn_permlane16_swap(bits(t), bits(u), false, false);
    return row_fsum(flt(c[0]) + flt(c[1]));
}
// Maximum over lanes l, l^16, l^32, l^48 combined with the row: all 64 lanes.
__device__ __forceinline__ uint32_t umax_all(uint32_t x) {
    const auto a = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    x = max(a[0], a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return row_umax(max(b[0], b[1]));
}
__device__ __forceinline__ uint32_t umax_xor32(uint32_t x) {
    const auto a = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return max(a[0], a[1]);
}

__device__ __forceinline__ void st16(uint8_t* p, uint32_t v) { *reinterpret_cast<uint16_t*>(p) = (uint16_t)v; }

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Exact part of a streaming decode for one (sequence, query head) row, by one
// wave: the residual tokens (bf16 K / V, at most 31, slots [B][Hkv][res_stride][D]).
// Lane l holds channels 2l and 2l + 1 (lanes >= D / 2 carry zeros).  Every
// window row is requested at once, one dword per lane and row, through buffer
// resources sized to the n_res valid slots (slots past it read as zeros, no
// branch); then one wave-wide sum per token.  The result: m, the sum of
// 2^(l - m) (l = q.k in log2 units) and x[c] = sum of 2^(l - m) v[2 lane + c].
constexpr int kResSlots = kGroup - 1;  // window slots that can hold a token
struct ResRows {
    uint32_t k[kResSlots], v[kResSlots];  // the lane's channel pair of every window row
    uint32_t q;                           // the lane's channel pair of the query
};
template <int D>
__device__ __forceinline__ void residual_load(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_res,
                                              const uint16_t* __restrict__ v_res, int res_stride, int n_res, int Hq,
                                              int Hkv, int row, int lane, ResRows& rr) {
    const int b = row / Hq, h = row % Hq;
    const int g = h / (Hq / Hkv);
    const size_t unit = (size_t)b * Hkv + g;
    const bool act = 2 * lane < D;
    const int off = act ? 4 * lane : 0;  // byte offset of the lane's channel pair within a row
    const int bytes = n_res * D * 2;
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(k_res + unit * res_stride * D), 0, bytes,
                                                      0x00020000);
    const auto rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(v_res + unit * res_stride * D), 0, bytes,
                                                      0x00020000);
#pragma unroll
    for (int t = 0; t < kResSlots; ++t) rr.k[t] = __builtin_amdgcn_raw_buffer_load_b32(rk, off + t * D * 2, 0, 0);
#pragma unroll
    for (int t = 0; t < kResSlots; ++t) rr.v[t] = __builtin_amdgcn_raw_buffer_load_b32(rv, off + t * D * 2, 0, 0);
    rr.q = act ? *reinterpret_cast<const uint32_t*>(q + (size_t)row * D + 2 * lane) : 0u;
}
__device__ __forceinline__ void residual_reduce(const ResRows& rr, int n_res, float scale_log2, float& m_out,
                                                float& l_out, float (&x)[2]) {
    const float q0 = bf16_bits_to_f32(rr.q & 0xFFFFu), q1 = bf16_bits_to_f32(rr.q >> 16);
    float l[kResSlots];
    float m = -INFINITY;
#pragma unroll
    for (int t = 0; t < kResSlots; ++t) {
        l[t] = -INFINITY;
        if (t < n_res) {  // wave-uniform
            const float d = fmaf(q0, bf16_bits_to_f32(rr.k[t] & 0xFFFFu), q1 * bf16_bits_to_f32(rr.k[t] >> 16));
            l[t] = dpp_sum<kWave>(d) * scale_log2;
            m = fmaxf(m, l[t]);
        }
    }
    float lsum = 0.0f;
    x[0] = 0.0f;
    x[1] = 0.0f;
#pragma unroll
    for (int t = 0; t < kResSlots; ++t) {
        if (t < n_res) {
            const float p = exp2f(l[t] - m);
            lsum += p;
            x[0] = fmaf(p, bf16_bits_to_f32(rr.v[t] & 0xFFFFu), x[0]);
            x[1] = fmaf(p, bf16_bits_to_f32(rr.v[t] >> 16), x[1]);
        }
    }
    m_out = m;
    l_out = lsum;
}

template <int D>
__device__ __forceinline__ void residual_part(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_res,
                                              const uint16_t* __restrict__ v_res, int res_stride, int n_res, int Hq,
                                              int Hkv, float scale_log2, int row, int lane, float& m_out,
                                              float& l_out, float (&x)[2]) {
    ResRows rr;
    residual_load<D>(q, k_res, v_res, res_stride, n_res, Hq, Hkv, row, lane, rr);
    residual_reduce(rr, n_res, scale_log2, m_out, l_out, x);
}

// Ticket-mode epilogue of a workgroup (all 64 NW threads): s_tp holds the NW
// waves' parts of (sequence, KV head) `unit`, each (head r) a row of D sums
// 2^(l - m) v, then m and the sum of 2^(l - m) (log2 units).  They are merged
// against their common maximum; with one workgroup per head (nwg == 1) the
// result is the output, otherwise it is part `wg` of the head in the
// workspace (ws_acc [unit][nwg][R][D], ws_ml [unit][nwg][R][2]) and the
// workgroup that takes the head's last ticket merges the nwg parts the same
// way, writes the output and resets the ticket to zero.  Empty parts (m = -inf,
// sum 0) get weight 0; the reference maximum is finite whenever one part is not
// empty.  With kWin, s_win (when not null) holds the exact part of a streaming
// cache's residual window in the same form, one row per head, and joins this
// workgroup's merge as one more part.
//
// The workgroups of a head may sit on different XCDs, whose L2 caches are not
// coherent with each other for ordinary accesses.  The parts are therefore
// written and read with agent-scope atomic stores and loads (device-coherent
// accesses that bypass the non-coherent caches) rather than behind full L2
// write-back / invalidate fences: every wave waits for its part stores to
// complete before the workgroup takes its ticket, and the last workgroup
// reads the parts only after its ticket has come back.
template <int D, int R, int NW, bool kWin>
__device__ __forceinline__ void ticket_merge(float (*s_tp)[R][D + 2], const float (*s_win)[D + 2], int* s_last,
                                             int unit, int wg, int nwg, float* __restrict__ ws_acc,
                                             float* __restrict__ ws_ml, __bf16* __restrict__ out,
                                             int32_t* __restrict__ tickets) {
    auto st_dev = [](float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
    auto ld_dev = [](const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
    constexpr int NTH = 64 * NW;
    __syncthreads();  // the waves' parts are in LDS
    for (int i = threadIdx.x; i < R * D; i += NTH) {
        const int r = i / D, c = i % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, s_tp[w][r][D]);
        if constexpr (kWin) {
            if (s_win) M = fmaxf(M, s_win[r][D]);  // workgroup-uniform
        }
        const float Ms = M == -INFINITY ? 0.0f : M;
        float L = 0.0f, O = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = exp2f(s_tp[w][r][D] - Ms);
            L = fmaf(s_tp[w][r][D + 1], f, L);
            O = fmaf(s_tp[w][r][c], f, O);
        }
        if constexpr (kWin) {
            if (s_win) {
                const float f = exp2f(s_win[r][D] - Ms);
                L = fmaf(s_win[r][D + 1], f, L);
                O = fmaf(s_win[r][c], f, O);
            }
        }
        const size_t row = (size_t)unit * R + r;
        if (nwg == 1) {
            out[row * D + c] = (__bf16)(O / L);
        } else {
            const size_t part = ((size_t)unit * nwg + wg) * R + r;
            st_dev(&ws_acc[part * D + c], O);
            if (c == 0) {
                st_dev(&ws_ml[part * 2 + 0], M);
                st_dev(&ws_ml[part * 2 + 1], L);
            }
        }
    }
    if (nwg == 1) return;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's part stores have completed at device scope ...
    __syncthreads();                // ... for every wave, before the ticket is taken
    if (threadIdx.x == 0) *s_last = atomicAdd(&tickets[unit], 1) == nwg - 1;
    __syncthreads();
    if (!*s_last) return;
    // One round of loads for everything the merge reads: every part's (m, sum)
    // (nwg * R <= 64 pairs, one per thread) and, per thread, its outputs' nwg
    // partial sums (at most kTicketMaxWorkgroups parts of ITER outputs); the
    // weights need the maximum over parts first, so the pairs go through LDS
    // (the LDS parts above are no longer needed).
    constexpr int ITER = (R * D + NTH - 1) / NTH;
    static_assert(kTicketMaxWorkgroups <= 8, "one batch of part loads");
    const size_t base = (size_t)unit * nwg * R;
    float m_i = 0.0f, l_i = 0.0f;
    const bool has_ml = (int)threadIdx.x < nwg * R;
    if (has_ml) {
        m_i = ld_dev(&ws_ml[(base + threadIdx.x) * 2]);
        l_i = ld_dev(&ws_ml[(base + threadIdx.x) * 2 + 1]);
    }
    float a[ITER][8];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int i = threadIdx.x + it * NTH;
        const int r = i / D, c = i % D;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            a[it][j] = (i < R * D && j < nwg) ? ld_dev(&ws_acc[(base + (size_t)j * R + r) * D + c]) : 0.0f;
    }
    float* s_ml = &s_tp[0][0][0];
    if (has_ml) {
        s_ml[2 * threadIdx.x] = m_i;
        s_ml[2 * threadIdx.x + 1] = l_i;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nwg * R; i += NTH) {  // weight of part i against its head's maximum
        const int r = i % R;
        float M = -INFINITY;
        for (int w = 0; w < nwg; ++w) M = fmaxf(M, s_ml[2 * (w * R + r)]);
        s_ml[2 * nwg * R + i] = exp2f(s_ml[2 * i] - (M == -INFINITY ? 0.0f : M));
    }
    __syncthreads();
    const float* s_f = s_ml + 2 * nwg * R;
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int i = threadIdx.x + it * NTH;
        if (i >= R * D) break;
        const int r = i / D, c = i % D;
        float L = 0.0f, O = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j < nwg) {
                const int pi = j * R + r;
                L = fmaf(s_ml[2 * pi + 1], s_f[pi], L);
                O = fmaf(a[it][j], s_f[pi], O);
            }
        }
        out[((size_t)unit * R + r) * D + c] = (__bf16)(O / L);
    }
    if (threadIdx.x == 0)  // zero again for the next call
        __hip_atomic_store(&tickets[unit], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Work item = (sequence, KV head, range of `chunk` tokens), numbered
// item = unit * splits + split with unit = b * Hkv + g.  Each wave is
// independent: it walks items blockIdx.x * 4 + wave, + 4 gridDim.x, ..., all
// 128-token steps of an item in order, and issues the first loads of its next
// item while it finishes the current one.
//
// With kTicket (a split head) the grid is one item per wave and a
// workgroup's NW waves hold NW consecutive token ranges of one (sequence, KV
// head): the NW parts are merged through LDS, each workgroup writes one part
// to the workspace (ws_splits = workgroups per KV head) and takes a ticket on
// the head; the workgroup that takes the last ticket merges the head's parts,
// writes the output and puts the ticket back to zero, so the whole decode is
// one launch with no spinning.  With kWin (a streaming cache's residual
// window: n_res rows of k_res / v_res, slots [B][Hkv][res_stride][D]) the
// last workgroup of each head also computes the window's exact part, waves
// NW - R .. NW - 1 one query head each after their own ranges (the last
// ranges, empty past the packed tokens), and merges it with its waves' parts.
template <int D, int R, int NW, bool kTicket, bool kWin>
__global__ __launch_bounds__(64 * NW, (!kTicket && R == 1) ? 4 : 1) void decode_partial_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ k_codes, const uint32_t* __restrict__ k_sz,
    const uint8_t* __restrict__ v_codes, const uint32_t* __restrict__ v_sz, int n, int tok_stride, int grp_stride,
    int chunk, int splits, int ws_splits, int direct, int n_items, float scale_log2, float* __restrict__ ws_acc,
    float* __restrict__ ws_ml, __bf16* __restrict__ out, const int32_t* __restrict__ counts,
    int32_t* __restrict__ tickets, const uint16_t* __restrict__ k_res, const uint16_t* __restrict__ v_res,
    int res_stride, int n_res) {
    static_assert(!kWin || kTicket, "the window part joins the one-launch merge");
    constexpr int NG = D / 32;  // 32-channel groups: key K blocks and value scale groups
    constexpr int NT = D / 16;  // 16-channel value tiles
    constexpr int GPL = NG * R / 4 > 1 ? NG * R / 4 : 1;  // value groups per lane in the weight prep
    __shared__ __align__(16) uint8_t s_qa[NW][4][R][4][128];   // wave, block, head, piece, K position
    __shared__ __align__(16) uint8_t s_wa[NW][R][NG][4][128];  // wave, head, value group, piece, K position
    __shared__ float s_z[NW][R][NG];
    // ticket mode: the waves' parts (sum 2^(l - m) v per channel, then m and the
    // sum of 2^(l - m)) and the last-ticket flag
    __shared__ float s_tp[kTicket ? NW : 1][R][D + 2];
    __shared__ float s_win[kWin ? R : 1][D + 2];  // the window part, in the same form
    __shared__ int s_last;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: keeps bases scalar
    const int lane = threadIdx.x % kWave;
    const int col = lane % 16, blk = lane / 16;
    const int myh = blk % R;  // head of this lane's MFMA result rows
    const int nwaves = gridDim.x * NW;
    int item = blockIdx.x * NW + wave;
    if (item >= n_items) return;  // wave-uniform; the kernel has no workgroup barrier
    // a device-side streaming step: the packed token count is read here (the
    // split plan covers the capacity n; ranges past the count are empty parts)
    if (counts) n = max(0, min(n, counts[0]));

    // never-written LDS positions must read as zero: key K positions >= D
    // (D < 128 only) and value piece 3 (every other byte is rewritten each step)
    if constexpr (D < 128) {
        uint32_t* za = reinterpret_cast<uint32_t*>(&s_qa[wave][0][0][0][0]);
        for (int i = lane; i < 4 * R * 4 * 128 / 4; i += kWave) za[i] = 0u;
    }
#pragma unroll
    for (int i = lane; i < R * NG * 32; i += kWave) {  // dword i % 32 of (head, group) row i / 32
        const int hg = i / 32;
        reinterpret_cast<uint32_t*>(&s_wa[wave][hg / NG][hg % NG][3][0])[i % 32] = 0u;
    }

    // Query channels c0, c0 + 2 of this lane sit at key K positions 2 lane,
    // 2 lane + 1 (lanes >= D/2 idle here).
    const bool qlane = lane < D / 2;
    const int c0 = qlane ? 32 * (lane / 16) + 16 * ((lane / 8) % 2) + 4 * (lane % 4) + (lane / 4) % 2 : 0;
    // Key B operand: the lane holds code words 2 blk, 2 blk + 1 (K positions
    // 32 blk + nibble) of one token; subtile j (0..7) of a step holds tokens
    // 32 (j/2) + 2 (j%2) + tm0 in its 16 columns, so the lane's two subtiles of
    // a block carry the tokens u, u + 2 that sit side by side in value K order.
    const int tm0 = 4 * (col / 2) + col % 2;
    const uint32_t koff = (uint32_t)(tm0 * (D / 4) + 8 * blk);
    // Value B operand: channel 16 T + col of block blk of the step, 8 bytes.
    const uint32_t voff = (uint32_t)((blk * D + col) * 8);
    // Weight prep: K position of token tm0 within a block (tm0 + 2 follows it),
    // value groups gbase .. gbase + GPL - 1 for head myh.
    const int kap = 16 * (col / 8) + 8 * (col % 2) + 2 * ((col / 2) % 4);
    const int gbase = (blk / R) * GPL;
    const bool wlane = gbase < NG;
    // A operand row lane % 16 = (head block, piece); piece k carries scale 16^-k
    const int ahd = (col / 4) % R, ap = col % 4;
    const int ascale = (127 - 4 * ap) * 0x01010101;

    // Everything one 128-token step needs from HBM.  Every load goes through a
    // buffer resource whose base is the step's first byte and whose size ends
    // at the last valid byte of the item's token range: lanes past the range
    // read zeros (codes 0, s = z = 0) with no branch, so the loads of the next
    // step land straight in the registers the current step has consumed.
    struct Stage {
        u32x4 kcw[4];   // code words of subtiles 2i, 2i + 1 as loaded (see load_keys)
        u32x4 kszw[4];  // scale / zero words of channels c0 - c0 % 4 .. + 3, per block
        uint2 vc[NT];
        uint32_t vsz[8][GPL];
    };
    auto rsrc = [](const void* base, int bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
    };
    auto tok_of = [&](int j) { return 32 * (j / 2) + 2 * (j % 2) + tm0; };  // token of subtile j in the step
    auto kc_off = [&](int j) { return koff + (uint32_t)((32 * (j / 2) + 2 * (j % 2)) * (D / 4)); };
    const uint32_t kszo = (uint32_t)(c0 * 4);
    const bool odd_row = (blk & 1) != 0;
    const uint32_t vszo = (uint32_t)((tm0 * NG + (wlane ? gbase : 0)) * 4);
    auto vsz_off = [&](int j, int i) { return vszo + (uint32_t)(((32 * (j / 2) + 2 * (j % 2)) * NG + i) * 4); };
    // position of a step: KV unit, step index, end of the item's token range
    struct Pos {
        int unit, step, t_end;
    };
    // Cache policy of the step loads: every packed byte is read once, so the
    // loads are non-temporal (nt).  Measured against the default policy: 3-6 %
    // faster per layer with one step per wave (the one-launch plans, small
    // batches), and 4-5 % faster over the 40-layer batch-1133 cache (40.9-41.3
    // against 42.9 ms per step).
    constexpr int kLoadPolicy = 2;
    auto load_keys = [&](const Pos& ps, Stage& st) {
        const int t0 = ps.step * kStep;
        const int nt = ps.t_end - t0;  // valid tokens from t0
        const auto rk = rsrc(k_codes + ((size_t)ps.unit * tok_stride + t0) * (D / 4), nt * (D / 4));
        const auto rs = rsrc(k_sz + ((size_t)ps.unit * grp_stride + t0 / kGroup) * D, (nt + kGroup - 1) / kGroup * D * 4);
        // Code words in 16-byte pieces: the lanes of an even 16-lane row take their
        // own 8 bytes of subtile 2i's token and the 8 the odd row beside them needs,
        // the lanes of an odd row those of subtile 2i + 1 (key_words() swaps the
        // halves when the step uses them, so the loads stay in flight until then).
        // Scale / zero words: one 16-byte load of channels c0 - c0 % 4 .. + 3 per
        // block (c0 and c0 + 2 among them).  Half as many load instructions as
        // 8-byte code and 4-byte word loads: the step loads alone went from 5.67
        // to 6.08 TB/s over a 40-layer batch-512 cache.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int off = odd_row ? (int)kc_off(2 * i + 1) - 8 : (int)kc_off(2 * i);
            st.kcw[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, kLoadPolicy));
        }
#pragma unroll
        for (int bk = 0; bk < 4; ++bk)
            st.kszw[bk] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)((kszo & ~15u) + bk * D * 4), 0, kLoadPolicy));
    };
    auto load_values = [&](const Pos& ps, Stage& st) {
        const int t0 = ps.step * kStep;
        const int nt = ps.t_end - t0;
        const auto rv = rsrc(v_codes + ((size_t)ps.unit * grp_stride + t0 / kGroup) * D * 8, (nt + kGroup - 1) / kGroup * D * 8);
        const auto rz = rsrc(v_sz + ((size_t)ps.unit * tok_stride + t0) * NG, nt * NG * 4);
#pragma unroll
        for (int T = 0; T < NT; ++T)
            st.vc[T] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rv, (int)(voff + 128 * T), 0, kLoadPolicy));
        // a token's GPL scale/zero words are adjacent: one load of GPL dwords
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if constexpr (GPL == 4) {
                const u32x4 w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rz, (int)vsz_off(j, 0), 0, kLoadPolicy));
#pragma unroll
                for (int i = 0; i < 4; ++i) st.vsz[j][i] = w[i];
            } else if constexpr (GPL == 2) {
                const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rz, (int)vsz_off(j, 0), 0, kLoadPolicy));
                st.vsz[j][0] = w[0];
                st.vsz[j][1] = w[1];
            } else {
                st.vsz[j][0] = __builtin_amdgcn_raw_buffer_load_b32(rz, (int)vsz_off(j, 0), 0, kLoadPolicy);
            }
        }
    };
    // the query of a KV unit: bf16 bits of channels c0, c0 + 2 for each of its R heads
    auto load_q = [&](int unit, uint32_t (&qb)[R][2]) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint16_t* qr = q + ((size_t)unit * R + r) * D;
            qb[r][0] = qr[c0];
            qb[r][1] = qr[c0 + 2];
        }
    };
    auto pos_of = [&](int it) {  // first step of an item (an empty range past n)
        const int t0 = (it % splits) * chunk;
        return Pos{it / splits, t0 / kStep, max(t0, min(n, t0 + chunk))};
    };

    // online-softmax state of this lane's head (uniform within its 16-lane row)
    float qk[R][2];
    float m_run, lacc;
    float acc[NT], zacc[GPL];

    // One step; the loads of the next position go out as soon as this step's
    // registers of the same kind are consumed.
    // The step's code words per subtile and scale / zero words per block, from
    // the 16-byte pieces load_keys fetched: one permlane16 swap per dword gives
    // each 16-lane row the half of the piece its neighbouring row loaded.
    auto key_words = [&](const Stage& st, uint2 (&kc)[8], uint32_t (&ksz)[4][2]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const auto s0 = __builtin_amdgcn_permlane16_swap(st.kcw[i][0], st.kcw[i][2], false, false);
            const auto s1 = __builtin_amdgcn_permlane16_swap(st.kcw[i][1], st.kcw[i][3], false, false);
            kc[2 * i] = make_uint2(s0[0], s1[0]);
            kc[2 * i + 1] = make_uint2(s0[1], s1[1]);
        }
#pragma unroll
        for (int bk = 0; bk < 4; ++bk) {
            ksz[bk][0] = (c0 & 1) ? st.kszw[bk][1] : st.kszw[bk][0];
            ksz[bk][1] = (c0 & 1) ? st.kszw[bk][3] : st.kszw[bk][2];
        }
    };

    auto process = [&](const Pos& ps, Stage& st, const Pos& nx) {
        const int t0 = ps.step * kStep;
        const int t_end = ps.t_end;
        uint2 kcs[8];
        uint32_t kszs[4][2];
        key_words(st, kcs, kszs);
        // ---- keys: fold each block's fp16 scales into the query ----
        float x[4][R][2], zp[4][R];
        uint32_t mxb[4][R];
#pragma unroll
        for (int bk = 0; bk < 4; ++bk) {
            const float s0 = half_bits_to_f32(kszs[bk][0] & 0xFFFFu), z0 = half_bits_to_f32(kszs[bk][0] >> 16);
            const float s1 = half_bits_to_f32(kszs[bk][1] & 0xFFFFu), z1 = half_bits_to_f32(kszs[bk][1] >> 16);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                x[bk][r][0] = qk[r][0] * s0;
                x[bk][r][1] = qk[r][1] * s1;
                mxb[bk][r] = __builtin_bit_cast(uint32_t, fmaxf(fabsf(x[bk][r][0]), fabsf(x[bk][r][1])));
                zp[bk][r] = fmaf(qk[r][0], z0, qk[r][1] * z1);
            }
        }
        // per (block, head): max |x| sets the pieces' power of two, sum q z is the block's score offset
        float bias[4][R], kmul[4][R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t mrow = umax4_rows(mxb[0][r], mxb[1][r], mxb[2][r], mxb[3][r]);
            const float zrow = fsum4_rows(zp[0][r], zp[1][r], zp[2][r], zp[3][r]);
#pragma unroll
            for (int bk = 0; bk < 4; ++bk) {
                const uint32_t e = piece_exp((uint32_t)__builtin_amdgcn_readlane((int)mrow, 16 * bk));
                bias[bk][r] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, zrow), 16 * bk));
                kmul[bk][r] = pow2_bits(e + 1);  // e2m1 holds code / 2
                uint32_t w[2];
                e4m3_pieces<4>(x[bk][r][0], x[bk][r][1], e, w);
                if (qlane) {
                    st16(&s_qa[wave][bk][r][0][2 * lane], w[0]);
                    st16(&s_qa[wave][bk][r][1][2 * lane], w[0] >> 16);
                    st16(&s_qa[wave][bk][r][2][2 * lane], w[1]);
                    st16(&s_qa[wave][bk][r][3][2 * lane], w[1] >> 16);
                }
            }
        }
        wave_sync_lds();
        // ---- keys: 8 MFMAs of 16 tokens, result rows = (head, piece) ----
        float sc[8];
#pragma unroll
        for (int bk = 0; bk < 4; ++bk) {
            const i32x8 A = a_operand(&s_qa[wave][bk][ahd][ap][16 * blk]);
            float km = kmul[bk][0], kb = bias[bk][0];
#pragma unroll
            for (int r = 1; r < R; ++r) {
                km = myh == r ? kmul[bk][r] : km;
                kb = myh == r ? bias[bk][r] : kb;
            }
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int j = 2 * bk + jj;
                const f32x4 c = mfma_f8_f4(A, codes_e2m1(kcs[j]), ascale);
                sc[j] = fmaf((c[0] + c[1]) + (c[2] + c[3]), km, kb);
            }
        }
        load_keys(nx, st);
        if (t0 + kStep > t_end) {  // wave-uniform: the step's tail is past the range
#pragma unroll
            for (int j = 0; j < 8; ++j) sc[j] = t0 + tok_of(j) < t_end ? sc[j] : -INFINITY;
        }
        // ---- online softmax over the step (a 16-lane row holds all 128 tokens of its head) ----
        float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
        const float m_new = fmaxf(m_run, fkey_inv(row_imax(fkey(mx))));
        if (__builtin_amdgcn_ballot_w64(m_new != m_run)) {  // wave-uniform
            const float alpha = exp2f(m_run - m_new);  // 0 on the first step (m_run = -inf)
            lacc *= alpha;
#pragma unroll
            for (int T = 0; T < NT; ++T) acc[T] *= alpha;
#pragma unroll
            for (int i = 0; i < GPL; ++i) zacc[i] *= alpha;
            m_run = m_new;
        }
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = __builtin_amdgcn_exp2f(sc[j] - m_run);  // 0 for masked tokens
            lacc += p[j];
        }
        // ---- values: weights w = p s per (token, value group), three e4m3 pieces ----
        float wv[8][GPL];
        float wmax = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
#pragma unroll
            for (int i = 0; i < GPL; ++i) {
                wv[j][i] = p[j] * half_bits_to_f32(st.vsz[j][i] & 0xFFFFu);
                zacc[i] = fmaf(p[j], half_bits_to_f32(st.vsz[j][i] >> 16), zacc[i]);
                wmax = fmaxf(wmax, wv[j][i]);
            }
        }
        // max over the lanes of this head: all 64 (R = 1), rows b and b + 2 (R = 2), the row (R = 4)
        uint32_t wmb = __builtin_bit_cast(uint32_t, wmax);
        if constexpr (R == 1) wmb = umax_all(wmb);
        else if constexpr (R == 2) wmb = row_umax(umax_xor32(wmb));
        else wmb = row_umax(wmb);
        const uint32_t ew = piece_exp(wmb);
#pragma unroll
        for (int bk = 0; bk < 4; ++bk) {
#pragma unroll
            for (int i = 0; i < GPL; ++i) {
                uint32_t w[2];
                e4m3_pieces<3>(wv[2 * bk][i], wv[2 * bk + 1][i], ew, w);
                if (wlane) {
                    uint8_t* dst = &s_wa[wave][myh][gbase + i][0][32 * bk + kap];
                    st16(dst, w[0]);
                    st16(dst + 128, w[0] >> 16);
                    st16(dst + 256, w[1]);
                }
            }
        }
        const float wmul = pow2_bits(ew + 1);
        wave_sync_lds();
        // ---- values: NT MFMAs of 16 channels x 128 tokens, result rows = (head, piece) ----
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
            const i32x8 A = a_operand(&s_wa[wave][ahd][gg][ap][16 * blk]);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int T = 2 * gg + tt;
                const f32x4 c = mfma_f8_f4(A, codes_e2m1(st.vc[T]), ascale);
                acc[T] = fmaf((c[0] + c[1]) + c[2], wmul, acc[T]);
            }
        }
        load_values(nx, st);
    };

    Stage st;
    Pos ps = pos_of(item);
    uint32_t qb[R][2];
    load_q(ps.unit, qb);
    load_keys(ps, st);
    load_values(ps, st);
    while (true) {
        const int split = item % splits;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            qk[r][0] = qlane ? bf16_bits_to_f32(qb[r][0]) * scale_log2 : 0.0f;  // log2 units
            qk[r][1] = qlane ? bf16_bits_to_f32(qb[r][1]) * scale_log2 : 0.0f;
        }
        m_run = -INFINITY;
        lacc = 0.0f;
#pragma unroll
        for (int T = 0; T < NT; ++T) acc[T] = 0.0f;
#pragma unroll
        for (int i = 0; i < GPL; ++i) zacc[i] = 0.0f;
        const int next_item = item + nwaves;
        const Pos first_next = pos_of(next_item);
        const int step_end = (ps.t_end + kStep - 1) / kStep;
        for (; ps.step < step_end; ++ps.step) {
            // next position: the next step, the next item's first step, or (after the
            // wave's last step) an empty range: the loads stay unconditional, and
            // with a zero-size buffer resource they return zeros without touching
            // memory
            const bool last = ps.step + 1 == step_end;
            const Pos nx = !last ? Pos{ps.unit, ps.step + 1, ps.t_end}
                                 : (next_item < n_items ? first_next : Pos{ps.unit, ps.step, ps.step * kStep});
            load_q(nx.unit, qb);
            process(ps, st, nx);
        }
        // ---- this item's result: row sums of l and of sum p z, out = acc + sum p z ----
        const float lsum = row_fsum(lacc);
#pragma unroll
        for (int i = 0; i < GPL; ++i) {
            const float zs = row_fsum(zacc[i]);
            if (col == 0 && wlane) s_z[wave][myh][gbase + i] = zs;
        }
        wave_sync_lds();
        if constexpr (kTicket) {
            if (blk < R) {
#pragma unroll
                for (int T = 0; T < NT; ++T) s_tp[wave][blk][16 * T + col] = acc[T] + s_z[wave][blk][T / 2];
                if (col == 0) {
                    s_tp[wave][blk][D] = m_run;
                    s_tp[wave][blk][D + 1] = lsum;
                }
            }
            const int wg = blockIdx.x % ws_splits;  // this workgroup's place among the head's
            const bool win = kWin && wg == ws_splits - 1;
            if constexpr (kWin) {
                if (win && wave >= NW - R) {  // wave-uniform: one query head per wave
                    const int r = wave - (NW - R);
                    const int nr = counts ? max(0, min(n_res, counts[1])) : n_res;
                    float m_r, l_r, x[2];
                    // with Hq = R and Hkv = 1 the row's KV unit is row / R
                    residual_part<D>(q, k_res, v_res, res_stride, nr, R, 1, scale_log2, ps.unit * R + r, lane, m_r,
                                     l_r, x);
                    if (2 * lane < D) {
                        s_win[r][2 * lane] = x[0];
                        s_win[r][2 * lane + 1] = x[1];
                    }
                    if (lane == 0) {
                        s_win[r][D] = m_r;
                        s_win[r][D + 1] = l_r;
                    }
                }
            }
            ticket_merge<D, R, NW, kWin>(s_tp, win ? s_win : nullptr, &s_last, ps.unit, wg, ws_splits, ws_acc, ws_ml,
                                         out, tickets);
            break;  // one item per wave
        }
        if (blk < R) {
            const size_t row = (size_t)ps.unit * R + blk;  // query head b * Hq + g * R + blk
#pragma unroll
            for (int T = 0; T < NT; ++T) {
                const float x = acc[T] + s_z[wave][blk][T / 2];
                if (direct)
                    out[row * D + 16 * T + col] = (__bf16)(x / lsum);
                else
                    ws_acc[(row * ws_splits + split) * D + 16 * T + col] = x;
            }
            if (!direct && col == 0) {
                ws_ml[(row * ws_splits + split) * 2 + 0] = m_run;
                ws_ml[(row * ws_splits + split) * 2 + 1] = lsum;
            }
        }
        wave_sync_lds();  // s_z is rewritten by the next item
        if (next_item >= n_items) break;
        item = next_item;
        ps = first_next;
    }
}

// Merge the token ranges of one (sequence, query head): the range maxima and
// weights 2^(m_s - M) are computed cooperatively and kept in LDS, then every
// thread (one channel) sums its partials with several loads in flight.  With
// k_res the workgroup has one more wave, which requests the window rows at the
// start and reduces them (residual_reduce) while the other waves sum the
// ranges; its part is merged last, as one more range.
constexpr int kMaxSplits = 256;
template <int D>
__global__ __launch_bounds__(D + kWave) void decode_combine_kernel(const float* __restrict__ ws_acc,
                                                                   const float* __restrict__ ws_ml, int splits,
                                                                   __bf16* __restrict__ out,
                                                                   const uint16_t* __restrict__ q,
                                                                   const uint16_t* __restrict__ k_res,
                                                                   const uint16_t* __restrict__ v_res, int res_stride,
                                                                   int n_res, int Hq, int Hkv, float scale_log2,
                                                                   const int32_t* __restrict__ counts) {
    constexpr int NW = D / kWave;
    __shared__ float s_w[kMaxSplits];
    __shared__ float s_part[2][NW];
    __shared__ float s_res[D + 2];  // window part: sum 2^(l - m) v per channel, then m, sum 2^(l - m)
    const int bh = blockIdx.x;
    const int t = threadIdx.x;
    const bool res = k_res != nullptr;  // then blockDim.x = D + kWave
    const bool win = t >= D;            // the window wave
    ResRows rr;
    if (win) {
        if (counts) n_res = max(0, min(n_res, counts[1]));
        residual_load<D>(q, k_res, v_res, res_stride, n_res, Hq, Hkv, bh, t - D, rr);
    }
    const float* ml = ws_ml + (size_t)bh * splits * 2;
    float m = -INFINITY;
    if (!win) {
        for (int s = t; s < splits; s += D) m = fmaxf(m, ml[2 * s]);
        m = dpp_max<kWave>(m);
        if (t % kWave == 0) s_part[0][t / kWave] = m;
    }
    __syncthreads();
    float M = s_part[0][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_part[0][w]);
    // weights are taken against Ms: with every range empty (M = -inf, a
    // streaming step with nothing packed yet) they are all 0, not NaN
    const float Ms = M == -INFINITY ? 0.0f : M;
    float l = 0.0f;
    if (!win) {
        for (int s = t; s < splits; s += D) {
            const float w = exp2f(ml[2 * s] - Ms);
            s_w[s] = w;
            l = fmaf(ml[2 * s + 1], w, l);
        }
        l = dpp_sum<kWave>(l);
        if (t % kWave == 0) s_part[1][t / kWave] = l;
    }
    __syncthreads();
    float o = 0.0f, L = 0.0f;
    if (!win) {
#pragma unroll
        for (int w = 0; w < NW; ++w) L += s_part[1][w];
        const float* a = ws_acc + (size_t)bh * splits * D + t;
        float o0 = 0.0f, o1 = 0.0f, o2 = 0.0f, o3 = 0.0f;
        int s = 0;
        for (; s + 4 <= splits; s += 4) {
            o0 = fmaf(a[(size_t)s * D], s_w[s], o0);
            o1 = fmaf(a[(size_t)(s + 1) * D], s_w[s + 1], o1);
            o2 = fmaf(a[(size_t)(s + 2) * D], s_w[s + 2], o2);
            o3 = fmaf(a[(size_t)(s + 3) * D], s_w[s + 3], o3);
        }
        for (; s < splits; ++s) o0 = fmaf(a[(size_t)s * D], s_w[s], o0);
        o = (o0 + o1) + (o2 + o3);
    } else {
        float m_r, l_r, x[2];
        residual_reduce(rr, n_res, scale_log2, m_r, l_r, x);
        const int lane = t - D;
        if (2 * lane < D) {
            s_res[2 * lane] = x[0];
            s_res[2 * lane + 1] = x[1];
        }
        if (lane == 0) {
            s_res[D] = m_r;
            s_res[D + 1] = l_r;
        }
    }
    if (res) {
        __syncthreads();  // the window part is in s_res
        if (!win) {
            // one more range: rescale both sides to the larger maximum (a factor
            // of 0 for an empty window, m = -inf)
            const float Mt = fmaxf(M, s_res[D]);
            const float a = M == -INFINITY ? 0.0f : exp2f(Ms - Mt), c = exp2f(s_res[D] - Mt);
            L = fmaf(L, a, s_res[D + 1] * c);
            o = fmaf(o, a, s_res[t] * c);
        }
    }
    if (!win) out[(size_t)bh * D + t] = (__bf16)(o / L);
}

// A streaming cache with nothing packed: the window's tokens are the whole
// attention set, one (sequence, query head) per wave, written as the output.
template <int D>
__global__ __launch_bounds__(64) void decode_residual_kernel(const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ k_res,
                                                             const uint16_t* __restrict__ v_res, int res_stride,
                                                             int n_res, int Hq, int Hkv, float scale_log2,
                                                             __bf16* __restrict__ out) {
    const int row = blockIdx.x;  // b * Hq + h
    const int lane = threadIdx.x;
    float m, lsum, x[2];
    residual_part<D>(q, k_res, v_res, res_stride, n_res, Hq, Hkv, scale_log2, row, lane, m, lsum, x);
    if (2 * lane < D) {
        out[(size_t)row * D + 2 * lane] = (__bf16)(x[0] / lsum);
        out[(size_t)row * D + 2 * lane + 1] = (__bf16)(x[1] / lsum);
    }
}

// Resident workgroups of a decode instantiation on the current device: the
// persistent grid is sized to it.  Host-side queries only, cached.
template <int D, int R>
int resident_workgroups() {
    static const int per_cu = [] {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_partial_kernel<D, R, 4, false, false>, 256, 0) != hipSuccess ||
            nb < 1)
            nb = 1;
        return nb;
    }();
    static std::atomic<int> cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int c = cus[dev].load(std::memory_order_relaxed);
    if (c <= 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1) c = 256;
        cus[dev].store(c, std::memory_order_relaxed);
    }
    return per_cu * c;
}

// Where a decode reads: the packed region (n tokens; strides of its layout)
// and an optional exact residual (n_res tokens of res_stride slots).
struct DecodeSrc {
    // with counts (device int32 {n_packed, n_res, ...}), n and n_res are upper
    // bounds and the kernels read the actual counts
    const uint8_t* k_codes;
    const uint32_t* k_sz;
    const uint8_t* v_codes;
    const uint32_t* v_sz;
    int n, tok_stride, grp_stride;
    const uint16_t* k_res;
    const uint16_t* v_res;
    int res_stride, n_res;
    const int32_t* counts;
};

template <int D, int R>
hipError_t launch_dr(const void* q, const DecodeSrc& src, int B, int Hq, int Hkv, float scale_log2, void* out,
                     void* ws, const DecodePlan& plan, hipStream_t stream) {
    const auto qq = static_cast<const uint16_t*>(q);
    const auto o = static_cast<__bf16*>(out);
    const bool res = src.n_res > 0;
    if (src.n <= 0) {  // the window alone: one part, written as the output
        hipLaunchKernelGGL((decode_residual_kernel<D>), dim3(B * Hq), dim3(kWave), 0, stream, qq, src.k_res,
                           src.v_res, src.res_stride, src.n_res, Hq, Hkv, scale_log2, o);
        return hipGetLastError();
    }
    // workspace: the tickets of split heads first (kTicketBytes, zero between
    // calls), then the parts
    int32_t* tickets = static_cast<int32_t*>(ws);
    float* ws_acc = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kTicketBytes);
    const int parts = plan.splits;
    const long items = (long)B * Hkv * plan.splits;
    if (plan.ticket && (res || !src.counts)) {
        // one launch: one item per wave, plan.nw ranges of a head per
        // workgroup, the last workgroup of each head merges (plan.splits %
        // plan.nw == 0); a residual window (res: always with device-side
        // counts) is computed and merged by the head's last workgroup
        const int nwg = parts / plan.nw;
        float* ws_ml = ws_acc + (size_t)B * Hq * nwg * D;
        auto go = [&](auto kernel, int nw) {
            hipLaunchKernelGGL(kernel, dim3((unsigned)(items / nw)), dim3(64 * nw), 0, stream, qq, src.k_codes,
                               src.k_sz, src.v_codes, src.v_sz, src.n, src.tok_stride, src.grp_stride, plan.chunk,
                               plan.splits, nwg, 0, (int)items, scale_log2, ws_acc, ws_ml, o, src.counts, tickets,
                               src.k_res, src.v_res, src.res_stride, src.n_res);
            return hipGetLastError();
        };
        if (res)
            return plan.nw == 8 ? go(decode_partial_kernel<D, R, 8, true, true>, 8)
                                : go(decode_partial_kernel<D, R, 4, true, true>, 4);
        return plan.nw == 8 ? go(decode_partial_kernel<D, R, 8, true, false>, 8)
                            : go(decode_partial_kernel<D, R, 4, true, false>, 4);
    }
    // packed ranges: plan.splits parts in the workspace (the output itself when
    // it is the only part); the window, if any, is computed and merged by the
    // merge kernel
    const bool direct = parts == 1 && !res;
    float* ws_ml = ws_acc + (size_t)B * Hq * parts * D;
    const long grid = std::min<long>((items + 3) / 4, resident_workgroups<D, R>());
    hipLaunchKernelGGL((decode_partial_kernel<D, R, 4, false, false>), dim3((unsigned)grid), dim3(256), 0, stream,
                       qq, src.k_codes, src.k_sz, src.v_codes, src.v_sz, src.n, src.tok_stride, src.grp_stride,
                       plan.chunk, plan.splits, parts, direct ? 1 : 0, (int)items, scale_log2, ws_acc, ws_ml, o,
                       src.counts, tickets, nullptr, nullptr, 0, 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || direct) return e;
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(B * Hq), dim3(D + (res ? kWave : 0)), 0, stream, ws_acc,
                       ws_ml, parts, o, qq,
                       res ? src.k_res : nullptr, src.v_res, src.res_stride, src.n_res, Hq, Hkv, scale_log2,
                       src.counts);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const void* q, const DecodeSrc& src, int B, int Hq, int Hkv, float scale_log2, void* out,
                    void* ws, const DecodePlan& plan, hipStream_t stream) {
    switch (Hq / Hkv) {
        case 1: return launch_dr<D, 1>(q, src, B, Hq, Hkv, scale_log2, out, ws, plan, stream);
        case 2: return launch_dr<D, 2>(q, src, B, Hq, Hkv, scale_log2, out, ws, plan, stream);
        case 4: return launch_dr<D, 4>(q, src, B, Hq, Hkv, scale_log2, out, ws, plan, stream);
        default: return hipErrorInvalidValue;
    }
}

// Split partials of the allocation-free decode entry point: a library-owned
// device array of kDecodeScratchBytes per GPU, held until the process ends.
// Host code never passes this name to a kernel (on the host it is only a
// stand-in symbol); decode_scratch() resolves its device address once per
// device and every launch takes that address.
__device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

}  // namespace

void* decode_scratch() {
    constexpr int kMaxDevices = 64;
    static std::atomic<void*> addr[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        // with the device current: this device's copy of the array
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        addr[dev].store(p, std::memory_order_release);  // concurrent first calls store the same address
    }
    return p;
}

DecodePlan decode_plan(int B, int Hq, int Hkv, int n_keep, int D) {
    (void)Hq;
    (void)D;
    const long units = (long)B * Hkv;
    const int steps = (n_keep + kStep - 1) / kStep;
    const long want = (4096 + units - 1) / units;  // aim for >= 4096 work items
    int splits = (int)(want < 1 ? 1 : (want > steps ? steps : want));
    if (splits > kMaxSplits - 4) splits = kMaxSplits - 4;  // room for a residual part in the merge
    int per = (steps + splits - 1) / splits;
    splits = (steps + per - 1) / per;
    bool ticket = false;
    int nw = 4;
    if (splits > 1) {
        // one launch: a split head takes whole workgroups of nw ranges (ranges
        // past the last token are empty parts, fewer than nw): one 4-wave
        // workgroup up to four ranges, 8-wave workgroups beyond, at most
        // kTicketMaxWorkgroups of them per head
        nw = splits <= 4 ? 4 : 8;
        const int rounded = (splits + nw - 1) / nw * nw;
        if (rounded <= nw * kTicketMaxWorkgroups) {
            splits = rounded;
            per = (steps + splits - 1) / splits;
            ticket = true;
        }
    }
    return {splits, per * kStep, ticket, nw};
}

size_t decode_ws_bytes(int B, int Hq, int D, const DecodePlan& plan) {
    // one-launch plans: one part per workgroup of nw ranges after the first
    // (a head in one workgroup merges in LDS); merge-kernel plans: one part
    // per range; a head of one range needs none
    const int parts =
        plan.ticket ? (plan.splits > plan.nw ? plan.splits / plan.nw : 0) : (plan.splits > 1 ? plan.splits : 0);
    return kTicketBytes + (size_t)B * Hq * parts * (D + 2) * sizeof(float);
}

size_t stream_decode_ws_bytes(int B, int Hq, int D, int n_packed, int n_res, const DecodePlan& plan) {
    const int parts = (n_packed > 0 ? plan.splits : 0) + (n_res > 0 ? 1 : 0);
    return kTicketBytes + (size_t)B * Hq * parts * (D + 2) * sizeof(float);
}

hipError_t launch_decode(const void* q, const uint8_t* k_codes, const uint32_t* k_sz, const uint8_t* v_codes,
                         const uint32_t* v_sz, int B, int Hq, int Hkv, int n_keep, int D, float sm_scale,
                         void* out, void* ws, const DecodePlan& plan, hipStream_t stream) {
    const float scale_log2 = sm_scale * kLog2e;
    const DecodeSrc src{k_codes, k_sz, v_codes, v_sz, n_keep, n_keep, (n_keep + kGroup - 1) / kGroup,
                        nullptr, nullptr, 0, 0, nullptr};
    if (D == 128) return launch_d<128>(q, src, B, Hq, Hkv, scale_log2, out, ws, plan, stream);
    return launch_d<64>(q, src, B, Hq, Hkv, scale_log2, out, ws, plan, stream);
}

hipError_t launch_stream_decode(const void* q, const uint8_t* k_codes, const uint32_t* k_sz, const uint8_t* v_codes,
                                const uint32_t* v_sz, int B, int Hq, int Hkv, int D, int cap, int n_packed,
                                const void* k_res, const void* v_res, int n_res, float sm_scale, void* out,
                                void* ws, const DecodePlan& plan, hipStream_t stream) {
    const float scale_log2 = sm_scale * kLog2e;
    const DecodeSrc src{k_codes, k_sz, v_codes, v_sz, n_packed, cap, cap / kGroup,
                        static_cast<const uint16_t*>(k_res), static_cast<const uint16_t*>(v_res), kGroup, n_res,
                        nullptr};
    if (D == 128) return launch_d<128>(q, src, B, Hq, Hkv, scale_log2, out, ws, plan, stream);
    return launch_d<64>(q, src, B, Hq, Hkv, scale_log2, out, ws, plan, stream);
}

hipError_t launch_stream_decode_counted(const void* q, const uint8_t* k_codes, const uint32_t* k_sz,
                                        const uint8_t* v_codes, const uint32_t* v_sz, int B, int Hq, int Hkv, int D,
                                        int cap, const int32_t* counts, const void* k_res, const void* v_res,
                                        float sm_scale, void* out, void* ws, const DecodePlan& plan,
                                        hipStream_t stream) {
    const float scale_log2 = sm_scale * kLog2e;
    // bounds: the whole capacity and a full window; the kernels read the counts
    const DecodeSrc src{k_codes, k_sz, v_codes, v_sz, cap, cap, cap / kGroup,
                        static_cast<const uint16_t*>(k_res), static_cast<const uint16_t*>(v_res), kGroup,
                        kGroup - 1, counts};
    if (D == 128) return launch_d<128>(q, src, B, Hq, Hkv, scale_log2, out, ws, plan, stream);
    return launch_d<64>(q, src, B, Hq, Hkv, scale_log2, out, ws, plan, stream);
}

}  // namespace minikv
