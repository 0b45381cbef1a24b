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
// Keys: the fp16 scale / zero of a 32-token group are folded into the query
// once per group (qs_c = q_c * s_c * scale * log2 e, bias = sum_c q_c z_c ...),
// so a token costs one multiply-add per channel on top of the unpack.
// Values: w = p_t * s is formed once per (token, 32-channel group) and the zero
// term is accumulated per group.  Softmax runs in the log2 domain (exp2).
//
// Work split: grid (splits, Hkv, B); a workgroup of 4 waves owns a range of
// `chunk` tokens (a multiple of 128) and walks it 128 tokens at a time, one
// 32-token group per wave.  A lane owns 16 channels (one 32-bit code word) of a
// token.  Partial (m, l, acc) per split go to the workspace; a small second
// kernel merges the splits by log-sum-exp and writes bf16.
#include "common.h"
#include "kernels.h"

namespace minikv {
namespace {

constexpr int kSub = 128;  // tokens per workgroup step: 4 waves x one 32-token group
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float code_at(uint32_t word, int c) {
    // channel c (0..15) of a 16-channel word: byte c/4, bits 2*(c%4)
    return (float)((word >> (8 * (c >> 2) + 2 * (c & 3))) & 3u);
}

template <int D, int R>
__global__ __launch_bounds__(256) void decode_partial_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ k_codes, const uint32_t* __restrict__ k_sz,
    const uint8_t* __restrict__ v_codes, const uint32_t* __restrict__ v_sz, int Hkv, int n, int chunk,
    float scale_log2, float* __restrict__ ws_acc, float* __restrict__ ws_ml) {
    constexpr int LPT = D / 16;      // lanes per token
    constexpr int TPW = kWave / LPT;  // tokens per wave step
    constexpr int G32 = kGroup / TPW;  // steps per 32-token group
    __shared__ float s_p[R][kSub];
    __shared__ float s_wmax[4][R];
    __shared__ float s_red[4][R][D];
    __shared__ float s_l[4][R];

    const int split = blockIdx.x;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int unit = b * Hkv + g;
    const int splits = gridDim.x;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int slot = lane / LPT;
    const int cc = lane % LPT;
    const int c0 = 16 * cc;
    const int G = (n + kGroup - 1) / kGroup;
    const int t_begin = split * chunk;
    const int t_end = min(n, t_begin + chunk);

    // query slice of this lane, pre-scaled into the log2 domain
    float qv[R][16];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint16_t* qp = q + ((size_t)(b * Hkv + g) * R + r) * D + c0;
        const u32x4 w0 = *reinterpret_cast<const u32x4*>(qp);
        const u32x4 w1 = *reinterpret_cast<const u32x4*>(qp + 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qv[r][2 * i] = bf16_bits_to_f32(w0[i] & 0xFFFFu) * scale_log2;
            qv[r][2 * i + 1] = bf16_bits_to_f32(w0[i] >> 16) * scale_log2;
            qv[r][8 + 2 * i] = bf16_bits_to_f32(w1[i] & 0xFFFFu) * scale_log2;
            qv[r][8 + 2 * i + 1] = bf16_bits_to_f32(w1[i] >> 16) * scale_log2;
        }
    }

    float m_run[R], acc[R][16], zacc[R], lacc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        m_run[r] = -INFINITY;
        zacc[r] = 0.0f;
        lacc[r] = 0.0f;
#pragma unroll
        for (int c = 0; c < 16; ++c) acc[r][c] = 0.0f;
    }

    for (int sub0 = t_begin; sub0 < t_end; sub0 += kSub) {
        // ---- keys: scores of this wave's 32-token group ----
        const int grp0 = sub0 + kGroup * wave;  // first token of the wave's group
        float wmax[R];
#pragma unroll
        for (int r = 0; r < R; ++r) wmax[r] = -INFINITY;
        if (grp0 < t_end) {
            const int gi = grp0 / kGroup;
            const uint32_t* szp = k_sz + ((size_t)unit * G + gi) * D + c0;
            float qs[R][16], bias[R];
#pragma unroll
            for (int r = 0; r < R; ++r) bias[r] = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x4 w = *reinterpret_cast<const u32x4*>(szp + 4 * i);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float s = half_bits_to_f32(w[e] & 0xFFFFu);
                    const float z = half_bits_to_f32(w[e] >> 16);
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        qs[r][4 * i + e] = qv[r][4 * i + e] * s;
                        bias[r] = fmaf(qv[r][4 * i + e], z, bias[r]);
                    }
                }
            }
#pragma unroll
            for (int st = 0; st < G32; ++st) {
                const int tl = slot + TPW * st;  // token within the group
                const int t = grp0 + tl;
                const bool valid = t < t_end;
                uint32_t word = 0;
                if (valid) word = *reinterpret_cast<const uint32_t*>(k_codes + ((size_t)unit * n + t) * (D / 4) + 4 * cc);
                float part[R];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float a = bias[r];
#pragma unroll
                    for (int c = 0; c < 16; ++c) a = fmaf(qs[r][c], code_at(word, c), a);
                    part[r] = a;
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float sc = group_sum<LPT>(part[r]);  // every lane takes part in the shuffle
                    sc = valid ? sc : -INFINITY;
                    if (cc == 0) s_p[r][kGroup * wave + tl] = sc;
                    wmax[r] = fmaxf(wmax[r], sc);
                }
            }
        } else {
            // no tokens for this wave: mark its slice empty
            for (int i = lane; i < kGroup; i += kWave)
#pragma unroll
                for (int r = 0; r < R; ++r) s_p[r][kGroup * wave + i] = -INFINITY;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float mx = wmax[r];
#pragma unroll
            for (int o = LPT; o < kWave; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
            if (lane == 0) s_wmax[wave][r] = mx;
        }
        __syncthreads();
        // ---- softmax bookkeeping (block-uniform) ----
        float alpha[R], m_new[R];
        bool rescale = false;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float ms = fmaxf(fmaxf(s_wmax[0][r], s_wmax[1][r]), fmaxf(s_wmax[2][r], s_wmax[3][r]));
            m_new[r] = fmaxf(m_run[r], ms);
            alpha[r] = exp2f(m_run[r] - m_new[r]);  // 0 on the first step (m_run = -inf)
            rescale |= m_new[r] != m_run[r];
            m_run[r] = m_new[r];
        }
        // probabilities of the 128 tokens
        for (int i = threadIdx.x; i < R * kSub; i += blockDim.x) {
            const int r = i / kSub, t = i % kSub;
            s_p[r][t] = exp2f(s_p[r][t] - m_new[r]);
        }
        if (rescale) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                zacc[r] *= alpha[r];
                lacc[r] *= alpha[r];
#pragma unroll
                for (int c = 0; c < 16; ++c) acc[r][c] *= alpha[r];
            }
        }
        __syncthreads();
        // ---- values ----
        if (grp0 < t_end) {
#pragma unroll
            for (int st = 0; st < G32; ++st) {
                const int tl = slot + TPW * st;
                const int t = grp0 + tl;
                if (t < t_end) {
                    const size_t row = (size_t)unit * n + t;
                    const uint32_t word = *reinterpret_cast<const uint32_t*>(v_codes + row * (D / 4) + 4 * cc);
                    const uint32_t szw = v_sz[row * (D / 32) + (cc >> 1)];
                    const float s = half_bits_to_f32(szw & 0xFFFFu);
                    const float z = half_bits_to_f32(szw >> 16);
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const float p = s_p[r][kGroup * wave + tl];
                        const float w = p * s;
                        zacc[r] = fmaf(p, z, zacc[r]);
                        if (cc == 0) lacc[r] += p;
#pragma unroll
                        for (int c = 0; c < 16; ++c) acc[r][c] = fmaf(w, code_at(word, c), acc[r][c]);
                    }
                }
            }
        }
        __syncthreads();
    }

    // ---- reduce the token slots of each wave, then the 4 waves ----
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            float x = acc[r][c] + zacc[r];
#pragma unroll
            for (int o = LPT; o < kWave; o <<= 1) x += __shfl_xor(x, o, kWave);
            if (slot == 0) s_red[wave][r][c0 + c] = x;
        }
        float l = lacc[r];
#pragma unroll
        for (int o = LPT; o < kWave; o <<= 1) l += __shfl_xor(l, o, kWave);
        if (lane == 0) s_l[wave][r] = l;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < R * D; i += blockDim.x) {
        const int r = i / D, d = i % D;
        const float x = s_red[0][r][d] + s_red[1][r][d] + s_red[2][r][d] + s_red[3][r][d];
        const size_t o = (((size_t)(b * Hkv + g) * R + r) * splits + split);
        ws_acc[o * D + d] = x;
        if (d == 0) {
            ws_ml[o * 2 + 0] = m_run[r];
            ws_ml[o * 2 + 1] = s_l[0][r] + s_l[1][r] + s_l[2][r] + s_l[3][r];
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
