// Heavy-hitter + recent-window selection of one (sequence, KV head) row by
// one workgroup: the device code of the selection kernel (select.hip), kept
// as a header so that another kernel can run a row's selection in place.
//
// Method: gptget.net summary of arXiv 2411.18077, 术语表 "adaptive KV" (keep
// the KV states chosen by importance) and 方法论 (2-bit quantisation combined
// with the adaptive policy).  Rule of this library: keep positions
// T-n_recent..T-1 and the n_heavy largest scores among positions < T-n_recent,
// equal scores going to the lower position; emit the union ascending.
//
// Each thread holds a contiguous run of candidate scores (in registers up to
// 32 per thread) as order-preserving uint32 keys.  An MSB-first radix select
// (4 passes of 8 bits, per-wave LDS histograms, the threshold digit found by
// one wave's prefix sum) finds the threshold key and how many threshold-equal
// keys to take; two block scans then compact the kept positions in ascending
// order.  Every decision is an integer comparison of fp32 bit patterns, so the
// result equals a sort of the same fp32 scores.
#pragma once

#include "common.h"

namespace minikv {
namespace sel {

constexpr int kHistStride = 257;  // one extra word per wave: sub-histograms start in different banks

// LDS of one row selection by NT threads
template <int NT>
struct Shared {
    uint32_t hist[NT / kWave * kHistStride];
    uint32_t wave[NT / kWave];
    uint32_t prefix, krem;
};

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);  // -0 and +0 compare equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the NT threads; *total receives the sum.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t* s_wave, uint32_t* total) {
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    uint32_t inc = x;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        uint32_t y = (uint32_t)__shfl_up((int)inc, o, kWave);
        if (lane >= o) inc += y;
    }
    if (lane == kWave - 1) s_wave[wave] = inc;
    __syncthreads();
    uint32_t wave_off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        uint32_t t = s_wave[w];
        wave_off += (w < wave) ? t : 0u;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return wave_off + inc - x;
}

// Selection of row srow (T_ctx fp32 scores) into orow (n_heavy + n_recent
// ascending positions), by all NT threads of the workgroup (every thread must
// call it).  ITEMS bounds the candidates per thread kept in registers
// (ITEMS > 32: re-read from L2 on each pass).
template <int ITEMS, int NT>
__device__ __forceinline__ void select_row(const float* __restrict__ srow, int T_ctx, int n_heavy, int n_recent,
                                           int32_t* __restrict__ orow, Shared<NT>& sh) {
    constexpr int NW = NT / kWave;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int n_cand = T_ctx - n_recent;
    const int per = (n_cand + NT - 1) / NT;
    const int begin = tid * per;
    // Rows of up to 32 keys per thread stay in registers; longer rows are
    // re-read from L2 on each pass (the register file would spill).
    constexpr bool kInRegs = ITEMS <= 32;
    uint32_t key_r[kInRegs ? ITEMS : 1];
    auto valid = [&](int i) { return i < per && begin + i < n_cand; };
    if constexpr (kInRegs) {
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) key_r[i] = valid(i) ? order_key(srow[begin + i]) : 0u;
    }
    auto key_at = [&](int i) -> uint32_t {
        if constexpr (kInRegs) return key_r[i];
        else return order_key(srow[begin + i]);
    };
    const int n_items = kInRegs ? ITEMS : per;  // constant trip count only for the register variant

    uint32_t prefix = 0, mask = 0, krem = (uint32_t)n_heavy;
    if (n_heavy > 0) {
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            for (int b = tid; b < NW * kHistStride; b += NT) sh.hist[b] = 0;
            __syncthreads();
            uint32_t* h = sh.hist + wave * kHistStride;
#pragma unroll
            for (int i = 0; i < n_items; ++i) {
                if (valid(i)) {
                    const uint32_t key = key_at(i);
                    if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & 255u], 1u);
                }
            }
            __syncthreads();
            // fold the per-wave histograms into wave 0's
            if (tid < 256) {
                uint32_t c = 0;
#pragma unroll
                for (int w = 0; w < NW; ++w) c += sh.hist[w * kHistStride + tid];
                sh.hist[tid] = c;
            }
            __syncthreads();
            if (tid < kWave) {
                // Threshold digit: the bucket d (counting down from 255) whose
                // count takes the running total from below krem to >= krem.
                // Lane l owns buckets 255 - 4l - j, j = 0..3; a wave prefix
                // sum over lanes gives each bucket the count above it.
                uint32_t c[4], incl[4], run = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    c[j] = sh.hist[255 - 4 * tid - j];
                    run += c[j];
                    incl[j] = run;
                }
                uint32_t scan = run;
#pragma unroll
                for (int o = 1; o < kWave; o <<= 1) {
                    const uint32_t y = (uint32_t)__shfl_up((int)scan, o, kWave);
                    if (tid >= o) scan += y;
                }
                const uint32_t above_lane = scan - run;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t above = above_lane + incl[j] - c[j];
                    if (above < krem && krem <= above + c[j]) {  // exactly one bucket
                        sh.prefix = prefix | ((uint32_t)(255 - 4 * tid - j) << shift);
                        sh.krem = krem - above;
                    }
                }
            }
            __syncthreads();
            prefix = sh.prefix;
            krem = sh.krem;
            mask |= 255u << shift;
            __syncthreads();
        }
    }
    // prefix: threshold key; krem: threshold-equal keys to take, lowest positions first.
    uint32_t gt = 0, eq = 0;
    if (n_heavy > 0) {
#pragma unroll
        for (int i = 0; i < n_items; ++i) {
            if (valid(i)) {
                const uint32_t key = key_at(i);
                gt += key > prefix;
                eq += key == prefix;
            }
        }
    }
    uint32_t tot;
    const uint32_t eq_before = block_exclusive_scan<NT>(eq, sh.wave, &tot);
    uint32_t take_eq = 0;
    if (krem > eq_before) take_eq = min(eq, krem - eq_before);
    const uint32_t off = block_exclusive_scan<NT>(gt + take_eq, sh.wave, &tot);
    if (n_heavy > 0) {
        uint32_t o = off, taken = 0;
#pragma unroll
        for (int i = 0; i < n_items; ++i) {
            if (valid(i)) {
                const uint32_t key = key_at(i);
                bool keep = key > prefix;
                if (key == prefix && taken < take_eq) {
                    keep = true;
                    ++taken;
                }
                if (keep && o < (uint32_t)n_heavy) orow[o++] = begin + i;  // bound holds by construction
            }
        }
    }
    for (int r = tid; r < n_recent; r += NT) orow[n_heavy + r] = n_cand + r;
}

}  // namespace sel
}  // namespace minikv
