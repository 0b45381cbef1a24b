// Single-query decode attention over the packed 2-bit cache.
//
// Method: paper-listing abstract (the 2-bit layer-discriminative cache serves
// inference) and the gptget.net summary, 方法详解 (per-channel keys, per-token
// values, compact layout).  For query head h on KV head g = h / R:
//   out = sum_t softmax_t(q . khat_t * scale) vhat_t,   xhat = code * s + z
// over the n_keep packed tokens.
//
// HBM-bound: the packed bytes of every kept token are read exactly once and
// dequantised in registers; the R query heads of a KV head share each read.
//
// Unpacking: a 32-bit code word holds 16 channels.  One v_and_or puts the two
// codes at bit position s of the word's 16-bit halves into the mantissas of two
// fp16 numbers whose exponent is chosen so that each equals exactly
// 2^(10-s) + code (s = 4, 6 or 8, i.e. offsets 64, 16, 4; the codes at other
// positions are first shifted there).  Ten instructions give eight fp16 pairs
// (channel j, channel j+8); v_dot2_f32_f16 then multiplies-and-adds two
// channels per instruction in fp32, and the known offsets are taken out again
// with the very same fp16 multipliers, so nothing but the multipliers is
// rounded.
// Keys: per 32-token group the wave folds the fp16 scale into the query,
// x = q * scale * log2 e * s, once per channel, splits it into two fp16 parts
// (hi = fp16(x), lo = fp16(x - hi): a single fp16 would put scores with large
// outlier channels outside the output tolerance) and shares them through LDS;
// a token then costs one unpack and two dot2 per channel pair, plus the fp32
// zero-point term sum_c q_c z_c computed once per group.
// Values: the code words of two tokens are interleaved with v_perm so that a
// dot2 with (p1 s1, p2 s2) accumulates both tokens into one channel; the zero
// term p z is accumulated per token.  Softmax runs in the log2 domain.
//
// Work split: grid (splits, Hkv, B); a workgroup of 4 waves owns a range of
// `chunk` tokens (a multiple of 128).  Each wave runs its own online softmax
// over the 32-token groups wave, wave + 4, ..., with every HBM load of the
// next group issued before the current group is processed (no workgroup
// barrier until the end); the 4 waves then merge by log-sum-exp.  Partial
// (m, l, acc) per split go to the workspace; a small second kernel merges the
// splits and writes bf16.
#include "common.h"
#include "kernels.h"

namespace minikv {
namespace {

constexpr int kSub = 128;  // tokens per workgroup step: 4 waves x one 32-token group
constexpr float kLog2e = 1.4426950408889634f;

// masks / exponent patterns for bit positions 4, 6, 8 of both 16-bit halves
constexpr uint32_t kM4 = 0x00300030u, kM6 = 0x00C000C0u, kM8 = 0x03000300u;
constexpr uint32_t kG4 = (21u << 10) | (21u << 26);  // 2^6  = 64
constexpr uint32_t kG6 = (19u << 10) | (19u << 26);  // 2^4  = 16
constexpr uint32_t kG8 = (17u << 10) | (17u << 26);  // 2^2  = 4
// offset carried by pair j (channels j and j+8 of a word)
__device__ __forceinline__ constexpr float pair_offset(int j) {
    return (j == 4 || j == 7) ? 4.0f : ((j == 1 || j == 3 || j == 6) ? 16.0f : 64.0f);
}

__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t g) { return (x & m) | g; }

// The six mask / exponent constants, held in registers: VOP3 on gfx9 takes no
// literal, so with literals the compiler splits each v_and_or_b32 in two.
struct UnpackConsts {
    uint32_t m4, m6, m8, g4, g6, g8;
};
__device__ __forceinline__ UnpackConsts unpack_consts() {
    uint32_t zero;  // a VGPR 0 the compiler cannot see through, so the constants stay in VGPRs
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    return {kM4 | zero, kM6 | zero, kM8 | zero, kG4 | zero, kG6 | zero, kG8 | zero};
}

// Eight fp16 pairs of a 16-channel code word: pair j = (off_j + code[j], off_j + code[j + 8]).
__device__ __forceinline__ void unpack16(uint32_t w, const UnpackConsts& k, uint32_t (&h)[8]) {
    const uint32_t xl = w << 4, xr = w >> 6;
    h[0] = and_or(xl, k.m4, k.g4);
    h[1] = and_or(xl, k.m6, k.g6);
    h[2] = and_or(w, k.m4, k.g4);
    h[3] = and_or(w, k.m6, k.g6);
    h[4] = and_or(w, k.m8, k.g8);
    h[5] = and_or(xr, k.m4, k.g4);
    h[6] = and_or(xr, k.m6, k.g6);
    h[7] = and_or(xr, k.m8, k.g8);
}

__device__ __forceinline__ f16x2 as_h2(uint32_t u) {
    f16x2 r;
    __builtin_memcpy(&r, &u, 4);
    return r;
}
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

template <int D, int R>
__global__ __launch_bounds__(256) void decode_partial_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ k_codes, const uint32_t* __restrict__ k_sz,
    const uint8_t* __restrict__ v_codes, const uint32_t* __restrict__ v_sz, int Hkv, int n, int chunk,
    float scale_log2, float* __restrict__ ws_acc, float* __restrict__ ws_ml) {
    constexpr int W16 = D / 16;          // 16-channel code words per token
    constexpr int VITEMS = (kGroup / 2) * W16 / kWave;  // values: (token pair, word) items per lane
    // per wave and head: four fp8 pieces of the scaled query, each in MFMA K order (128 bytes)
    __shared__ __align__(16) uint8_t s_qa[4][R][4][128];
    __shared__ float s_p[4][R][kGroup];        // per wave: probabilities of its group
    __shared__ float s_red[4][R][D];
    __shared__ float s_ml[4][R][2];

    const int split = blockIdx.x;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int unit = b * Hkv + g;
    const int splits = gridDim.x;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: keeps group bases scalar
    const int lane = threadIdx.x % kWave;
    const int G = (n + kGroup - 1) / kGroup;
    const int t_begin = split * chunk;
    const int t_end = min(n, t_begin + chunk);
    const int gi_begin = t_begin / kGroup;
    const int gi_end = (t_end + kGroup - 1) / kGroup;

    // Query channels of this lane: the pair (c0, c0 + 2) sits at MFMA K positions 2 lane, 2 lane + 1
    // (lanes >= D/2 idle here).  Pre-scaled to log2 units.
    const bool qlane = lane < D / 2;
    const int c0 = qlane ? 32 * (lane / 16) + 16 * ((lane / 8) % 2) + 4 * (lane % 4) + (lane / 4) % 2 : 0;
    float qk[R][2];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint16_t* qr = q + ((size_t)(b * Hkv + g) * R + r) * D;
        qk[r][0] = qlane ? bf16_bits_to_f32(qr[c0]) * scale_log2 : 0.0f;
        qk[r][1] = qlane ? bf16_bits_to_f32(qr[c0 + 2]) * scale_log2 : 0.0f;
    }
    // keys as MFMA B operand: lane holds token 16 j + lane % 16, code words 2 (lane / 16), + 1
    const bool kact = lane / 16 < D / 32;
    const uint32_t koff = (uint32_t)((lane % 16) * (D / 4) + 8 * (lane / 16));
    // query pieces as MFMA A operand: row lane % 16 = (head block, piece)
    const int arow = lane % 16;
    const uint8_t* a_src = &s_qa[wave][(arow / 4) % R][arow % 4][16 * (lane / 16)];
    const int myh = (lane / 16) % R;  // head of this lane's score rows
    const UnpackConsts uk = unpack_consts();
    if (D < 128) {  // K positions past D stay zero
        for (int i = lane; i < R * 4 * 128 / 4; i += kWave)
            reinterpret_cast<uint32_t*>(&s_qa[wave][0][0][0])[i] = 0u;
    }

    // Everything one 32-token group needs from HBM, loaded one group ahead.
    struct Stage {
        uint2 kc[2];
        uint32_t ksz[2];
        uint32_t vc[VITEMS][2];
        uint32_t vsz[VITEMS][2];
    };
    // Lane byte offsets inside a group (constant, unsigned 32-bit) added to
    // wave-uniform group bases, so loads use scalar base + vector offset.
    uint32_t vcoff[VITEMS][2], vsoff[VITEMS][2];
#pragma unroll
    for (int it = 0; it < VITEMS; ++it) {
        const int item = lane + kWave * it;
        const int cc = item % W16, pr = item / W16;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            vcoff[it][e] = (uint32_t)((2 * pr + e) * (D / 4) + 4 * cc);
            vsoff[it][e] = (uint32_t)(((2 * pr + e) * (D / 32) + (cc >> 1)) * 4);
        }
    }
    auto ld32 = [](const uint8_t* base, uint32_t off) {
        return *reinterpret_cast<const uint32_t*>(base + off);
    };
    auto ld64 = [](const uint8_t* base, uint32_t off) {
        return *reinterpret_cast<const uint2*>(base + off);
    };
    auto load_stage = [&](int gi, Stage& st) {
        const int grp0 = gi * kGroup;
        const size_t row0 = (size_t)unit * n + grp0;
        const uint8_t* kcb = k_codes + row0 * (D / 4);
        const uint8_t* vcb = v_codes + row0 * (D / 4);
        const uint8_t* vsb = reinterpret_cast<const uint8_t*>(v_sz + row0 * (D / 32));
        const uint32_t* kszb = k_sz + ((size_t)unit * G + gi) * D;
        st.ksz[0] = kszb[c0];
        st.ksz[1] = kszb[c0 + 2];
        if (grp0 + kGroup <= t_end) {  // wave-uniform: the whole group is in range
#pragma unroll
            for (int j = 0; j < 2; ++j)
                st.kc[j] = kact ? ld64(kcb, koff + (uint32_t)(j * 16 * (D / 4))) : make_uint2(0u, 0u);
#pragma unroll
            for (int it = 0; it < VITEMS; ++it) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    st.vc[it][e] = ld32(vcb, vcoff[it][e]);
                    st.vsz[it][e] = ld32(vsb, vsoff[it][e]);
                }
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int t = grp0 + 16 * j + lane % 16;
            st.kc[j] = kact && t < t_end ? ld64(kcb, koff + (uint32_t)(j * 16 * (D / 4))) : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int it = 0; it < VITEMS; ++it) {
            const int item = lane + kWave * it;
            const int pr = item / W16;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const bool in = grp0 + 2 * pr + e < t_end;
                st.vc[it][e] = in ? ld32(vcb, vcoff[it][e]) : 0u;
                st.vsz[it][e] = in ? ld32(vsb, vsoff[it][e]) : 0u;  // s = z = 0 adds nothing
            }
        }
    };

    // online-softmax state of this wave (m wave-uniform; l, acc per lane)
    // a lane's value items all use the same code word (item % W16 == lane % W16), so one accumulator set
    float m_run[R], lacc[R], acc[R][16], wsum[R], zacc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        m_run[r] = -INFINITY;
        lacc[r] = 0.0f;
        wsum[r] = 0.0f;
        zacc[r] = 0.0f;
#pragma unroll
        for (int c = 0; c < 16; ++c) acc[r][c] = 0.0f;
    }

    auto process = [&](int gi, const Stage& st) {
        const int grp0 = gi * kGroup;
        // ---- keys: fold the group's fp16 scales into the query, split into fp8 pieces ----
        const float s0 = half_bits_to_f32(st.ksz[0] & 0xFFFFu), z0 = half_bits_to_f32(st.ksz[0] >> 16);
        const float s1 = half_bits_to_f32(st.ksz[1] & 0xFFFFu), z1 = half_bits_to_f32(st.ksz[1] >> 16);
        float bias[R], kmul[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float x0 = qk[r][0] * s0, x1 = qk[r][1] * s1;
            // common power of two putting max |x| in [128, 256): every piece stays finite in e4m3
            const float mx = dpp_max<kWave>(fmaxf(fabsf(x0), fabsf(x1)));
            const int sig = 8 - __builtin_amdgcn_readfirstlane(__builtin_amdgcn_frexp_expf(mx));
            x0 = __builtin_amdgcn_ldexpf(x0, sig);
            x1 = __builtin_amdgcn_ldexpf(x1, sig);
            uint32_t p01 = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
            f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8(p01, false);
            x0 -= f[0];
            x1 -= f[1];
            p01 = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, p01, true);
            f = __builtin_amdgcn_cvt_pk_f32_fp8(p01, true);
            x0 -= f[0];
            x1 -= f[1];
            uint32_t p23 = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
            f = __builtin_amdgcn_cvt_pk_f32_fp8(p23, false);
            x0 -= f[0];
            x1 -= f[1];
            p23 = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, p23, true);
            if (qlane) {
                *reinterpret_cast<uint16_t*>(&s_qa[wave][r][0][2 * lane]) = (uint16_t)p01;
                *reinterpret_cast<uint16_t*>(&s_qa[wave][r][1][2 * lane]) = (uint16_t)(p01 >> 16);
                *reinterpret_cast<uint16_t*>(&s_qa[wave][r][2][2 * lane]) = (uint16_t)p23;
                *reinterpret_cast<uint16_t*>(&s_qa[wave][r][3][2 * lane]) = (uint16_t)(p23 >> 16);
            }
            bias[r] = dpp_sum<kWave>(fmaf(qk[r][0], z0, qk[r][1] * z1));
            kmul[r] = __builtin_amdgcn_ldexpf(2.0f, -sig);  // fp4 holds code / 2
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // ---- keys: scores of the group's 32 tokens, two 16-token MFMAs (rows = head x piece) ----
        i32x8 A;
        {
            const u32x4 lo = *reinterpret_cast<const u32x4*>(a_src);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(a_src + 64);
            A = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
        float km = kmul[0], kb = bias[0];
#pragma unroll
        for (int r = 1; r < R; ++r) {
            km = myh == r ? kmul[r] : km;
            kb = myh == r ? bias[r] : kb;
        }
        float sc[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t w0 = st.kc[j].x, w1 = st.kc[j].y;
            const i32x8 Bk = {(int)(w0 & 0x33333333u), (int)((w0 >> 2) & 0x33333333u),
                              (int)(w1 & 0x33333333u), (int)((w1 >> 2) & 0x33333333u), 0, 0, 0, 0};
            const f32x4 c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bk, f32x4{0.0f, 0.0f, 0.0f, 0.0f},
                                                                             0, 4, 0, 0x7F7F7F7F, 0, 0x7F7F7F7F);
            sc[j] = fmaf((c[0] + c[1]) + (c[2] + c[3]), km, kb);
        }
        if (grp0 + kGroup > t_end) {  // wave-uniform: the group's tail is past the range
#pragma unroll
            for (int j = 0; j < 2; ++j) sc[j] = grp0 + 16 * j + lane % 16 < t_end ? sc[j] : -INFINITY;
        }
        // ---- softmax bookkeeping for this wave (wave-uniform per head) ----
        const float rowmax = dpp_max<16>(fmaxf(sc[0], sc[1]));
        float m_new[R];
        bool rescale = false;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float mx = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rowmax), 16 * r));
            m_new[r] = fmaxf(m_run[r], mx);
            rescale |= m_new[r] != m_run[r];
        }
        float mm = m_new[0];
#pragma unroll
        for (int r = 1; r < R; ++r) mm = myh == r ? m_new[r] : mm;
        // probabilities of the group's tokens, once per token (0 for masked tokens)
        if (lane < 16 * R) {
#pragma unroll
            for (int j = 0; j < 2; ++j) s_p[wave][myh][16 * j + lane % 16] = __builtin_amdgcn_exp2f(sc[j] - mm);
        }
        // probabilities of the group's tokens, once per token (0 for masked tokens)
        if (rescale) {  // wave-uniform
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float alpha = exp2f(m_run[r] - m_new[r]);  // 0 on the first group (m_run = -inf)
                lacc[r] *= alpha;
                wsum[r] *= alpha;
                zacc[r] *= alpha;
#pragma unroll
                for (int c = 0; c < 16; ++c) acc[r][c] *= alpha;
                m_run[r] = m_new[r];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // ---- values: token pairs ----
#pragma unroll
        for (int it = 0; it < VITEMS; ++it) {
            const int item = lane + kWave * it;
            const int cc = item % W16, pr = item / W16;
            const uint32_t plo = __builtin_amdgcn_perm(st.vc[it][1], st.vc[it][0], 0x05040100u);
            const uint32_t phi = __builtin_amdgcn_perm(st.vc[it][1], st.vc[it][0], 0x07060302u);
            uint32_t hl[8], hh[8];
            unpack16(plo, uk, hl);  // pair j: (token 0 channel j, token 1 channel j)
            unpack16(phi, uk, hh);  // pair j: (token 0 channel j+8, token 1 channel j+8)
            const float sA = half_bits_to_f32(st.vsz[it][0] & 0xFFFFu), zA = half_bits_to_f32(st.vsz[it][0] >> 16);
            const float sB = half_bits_to_f32(st.vsz[it][1] & 0xFFFFu), zB = half_bits_to_f32(st.vsz[it][1] >> 16);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float pA = s_p[wave][r][2 * pr];
                const float pB = s_p[wave][r][2 * pr + 1];
                f16x2 wv;
                wv[0] = (_Float16)(pA * sA);
                wv[1] = (_Float16)(pB * sB);
                uint32_t wu;
                __builtin_memcpy(&wu, &wv, 4);
                wsum[r] = dot2(wu, 0x3C003C00u, wsum[r]);  // exact sum of the fp16 weights
                zacc[r] = fmaf(pA, zA, fmaf(pB, zB, zacc[r]));
                if (cc == 0) lacc[r] += pA + pB;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    acc[r][j] = dot2(wu, hl[j], acc[r][j]);
                    acc[r][8 + j] = dot2(wu, hh[j], acc[r][8 + j]);
                }
            }
        }
    };

    // each wave walks groups wave, wave + 4, ... of this split, one group prefetched
    // (a second prefetched group costs more in occupancy than it gains)
    {
        Stage A, Bst;
        int gi = gi_begin + wave;
        if (gi < gi_end) load_stage(gi, A);
        while (gi < gi_end) {
            if (gi + 4 < gi_end) load_stage(gi + 4, Bst);
            process(gi, A);
            gi += 4;
            if (gi >= gi_end) break;
            if (gi + 4 < gi_end) load_stage(gi + 4, A);
            process(gi, Bst);
            gi += 4;
        }
    }

    // ---- this wave's partial: remove the unpack offsets, reduce lanes holding the same word ----
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float l = lacc[r];
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) l += __shfl_xor(l, o, kWave);
        if (lane == 0) {
            s_ml[wave][r][0] = m_run[r];
            s_ml[wave][r][1] = l;
        }
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            float x = acc[r][c] - pair_offset(c & 7) * wsum[r] + zacc[r];
#pragma unroll
            for (int o = W16; o < kWave; o <<= 1) x += __shfl_xor(x, o, kWave);
            if (lane < W16) s_red[wave][r][16 * lane + c] = x;
        }
    }
    __syncthreads();
    // ---- merge the 4 waves (log-sum-exp) into this split's partial ----
    for (int i = threadIdx.x; i < R * D; i += blockDim.x) {
        const int r = i / D, d = i % D;
        const float M = fmaxf(fmaxf(s_ml[0][r][0], s_ml[1][r][0]), fmaxf(s_ml[2][r][0], s_ml[3][r][0]));
        float x = 0.0f, L = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float f = exp2f(s_ml[w][r][0] - M);  // 0 for a wave that saw no tokens
            x = fmaf(s_red[w][r][d], f, x);
            L = fmaf(s_ml[w][r][1], f, L);
        }
        const size_t o = (((size_t)(b * Hkv + g) * R + r) * splits + split);
        ws_acc[o * D + d] = x;
        if (d == 0) {
            ws_ml[o * 2 + 0] = M;
            ws_ml[o * 2 + 1] = L;
        }
    }
}

// Merge the splits of one (sequence, query head): log-sum-exp weights, bf16 out.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const float* __restrict__ ws_acc,
                                                           const float* __restrict__ ws_ml, int splits,
                                                           __bf16* __restrict__ out) {
    const int bh = blockIdx.x;
    const int d = threadIdx.x;
    const float* ml = ws_ml + (size_t)bh * splits * 2;
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, ml[2 * s]);
    float L = 0.0f, o = 0.0f;
    for (int s = 0; s < splits; ++s) {
        const float w = exp2f(ml[2 * s] - M);
        L = fmaf(ml[2 * s + 1], w, L);
        o = fmaf(ws_acc[((size_t)bh * splits + s) * D + d], w, o);
    }
    out[(size_t)bh * D + d] = (__bf16)(o / L);
}

template <int D, int R>
hipError_t launch_dr(const void* q, const uint8_t* k_codes, const uint32_t* k_sz, const uint8_t* v_codes,
                     const uint32_t* v_sz, int B, int Hq, int Hkv, int n, float scale_log2, void* out,
                     void* ws, const DecodePlan& plan, hipStream_t stream) {
    float* ws_acc = static_cast<float*>(ws);
    float* ws_ml = ws_acc + (size_t)B * Hq * plan.splits * D;
    hipLaunchKernelGGL((decode_partial_kernel<D, R>), dim3(plan.splits, Hkv, B), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q), k_codes, k_sz, v_codes, v_sz, Hkv, n, plan.chunk,
                       scale_log2, ws_acc, ws_ml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(B * Hq), dim3(D), 0, stream, ws_acc, ws_ml,
                       plan.splits, static_cast<__bf16*>(out));
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const void* q, const uint8_t* k_codes, const uint32_t* k_sz, const uint8_t* v_codes,
                    const uint32_t* v_sz, int B, int Hq, int Hkv, int n, float scale_log2, void* out,
                    void* ws, const DecodePlan& plan, hipStream_t stream) {
    switch (Hq / Hkv) {
        case 1: return launch_dr<D, 1>(q, k_codes, k_sz, v_codes, v_sz, B, Hq, Hkv, n, scale_log2, out, ws, plan, stream);
        case 2: return launch_dr<D, 2>(q, k_codes, k_sz, v_codes, v_sz, B, Hq, Hkv, n, scale_log2, out, ws, plan, stream);
        case 4: return launch_dr<D, 4>(q, k_codes, k_sz, v_codes, v_sz, B, Hq, Hkv, n, scale_log2, out, ws, plan, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

DecodePlan decode_plan(int B, int Hkv, int n_keep) {
    const long units = (long)B * Hkv;
    const int max_splits = (n_keep + kSub - 1) / kSub;
    long want = (2048 + units - 1) / units;  // aim for >= 8 workgroups per CU
    int splits = (int)(want < 1 ? 1 : (want > max_splits ? max_splits : want));
    int chunk = (n_keep + splits - 1) / splits;
    chunk = (chunk + kSub - 1) / kSub * kSub;
    splits = (n_keep + chunk - 1) / chunk;
    return {splits, chunk};
}

size_t decode_ws_bytes(int B, int Hq, int D, const DecodePlan& plan) {
    return (size_t)B * Hq * plan.splits * (D + 2) * sizeof(float);
}

hipError_t launch_decode(const void* q, const uint8_t* k_codes, const uint32_t* k_sz, const uint8_t* v_codes,
                         const uint32_t* v_sz, int B, int Hq, int Hkv, int n_keep, int D, float sm_scale,
                         void* out, void* ws, const DecodePlan& plan, hipStream_t stream) {
    const float scale_log2 = sm_scale * kLog2e;
    if (D == 128)
        return launch_d<128>(q, k_codes, k_sz, v_codes, v_sz, B, Hq, Hkv, n_keep, scale_log2, out, ws, plan, stream);
    return launch_d<64>(q, k_codes, k_sz, v_codes, v_sz, B, Hq, Hkv, n_keep, scale_log2, out, ws, plan, stream);
}

}  // namespace minikv
