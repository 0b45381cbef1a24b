// Selective flash attention, pass 1: causal attention with per-row log-sum-exp.
//
// Method: paper-listing abstract (kernels that keep the 2-bit cache compatible
// with FlashAttention) and gptget.net summary, 方法详解 (selective flash
// attention built from a second kernel, memory kept low).  This pass computes
//   o[i]   = sum_{j<=i} softmax_j(q_i . k_j * scale) v_j
//   lse[i] = log sum_{j<=i} exp(q_i . k_j * scale)
// in one sweep over the keys with an online softmax; the second kernel
// (window_scores.hip) reuses lse to turn the last rows' logits into
// probabilities without storing any T x T matrix.
//
// gfx950 design: a workgroup of 8 waves owns 256 query rows (32 per wave) and
// streams 64-key tiles of K and V through two LDS stages (register-prefetched;
// one barrier per tile).  Workgroups are ordered XCD-aware so the K/V prefix a
// head's query blocks share stays in one L2.  Each wave software-pipelines its
// tiles: while the softmax of tile t runs on the VALU, the matrix cores take
// the PV product of tile t-1 and the QK^T product of tile t+1, one MFMA per
// slot with a share of the vector work between them, so that the VALU and the
// matrix cores of a SIMD work side by side.  Each wave computes S^T = K Q^T with
// bf16 MFMA 32x32x16, so an accumulator column is one query: a lane owns the
// softmax state (running max, partial sum) of its query, and the row max needs
// one permlane32 swap.  P^T is already in the B-operand layout of the second
// product O^T = V^T P^T.  V is transposed on its way into LDS (each thread
// packs the fp16 values of two adjacent keys into one dword), so every V^T
// operand is a single 16-byte LDS read.  The key order inside a
// 32-key block is permuted (phys) so that accumulator register v of a lane is
// key 16*half + v, which makes both operand layouts line up without shuffles.
// Causal: tiles above the diagonal are never loaded; only tiles that cross it
// apply the mask.  Query blocks are issued longest-first.  O leaves through LDS,
// so every global store writes whole 128-byte half rows.
//
// Single-pass selective attention: when each KV head has one query head and
// the W <= 32 observation rows all fall in a head's last query block, the
// workgroup that finishes that block computes the head's window scores right
// away (window_mass.h, the second pass's arithmetic): the rows' lse values
// stay in LDS, the 8 waves split the head's keys, which the block has just
// streamed and the Infinity Cache still holds, and no second launch is needed.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "window_mass.h"

namespace minikv {
namespace {

#ifndef MINIKV_FA_WAVES
#define MINIKV_FA_WAVES 8
#endif
constexpr int kFaWaves = MINIKV_FA_WAVES;  // waves per workgroup, 32 query rows each
constexpr int kXcds = 8;                    // MI355X: 8 XCDs of 32 CUs, each with its own L2
constexpr int kBN = 64;   // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// logical accumulator row r of a 32-key block -> physical key within the block
__device__ __forceinline__ int phys_key(int r) { return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }

// inverse of phys_key: LDS row (lane order) of key r of a 32-key block
__device__ __forceinline__ int key_lane(int r) { return (r & 3) | (((r >> 4) & 1) << 2) | (((r >> 2) & 3) << 3); }

// Staged K tile: the keys of each 32-key block are stored in the order the
// lanes read them (row key_lane(r) holds key r), with rows padded by 16 bytes,
// so a K-operand read (32 consecutive rows, one 16-byte chunk: lane l starts
// at bank 4 l mod 64 within its half) touches distinct banks in every pass,
// and every operand address is one lane constant plus an immediate.
template <int D>
constexpr int kKStride = D + 8;  // elements per staged K row

// Staged V^T tile.  Element (key, d) with key = 32 bk + 16 half + 8 s + i and
// d = 8 c + e, c = 8 c_hi + c_lo, sits in line
//   ((bk * 2 + s) * (D / 64) + c_hi) * 8 + e
// at byte 16 (c_lo + 8 half) + 2 i.  Lines are padded from 256 to 320 bytes.
// The 64 lanes of a transposed-store dword write (fixed e, varying c_lo, half
// and key pair) write 64 dwords of one line.  A 16-byte read is served in four
// passes of 16 lanes: one half of the wave, and within it the four lane quads
// whose quad index (lane / 4 mod 8) has the same bit parity.  In a PV operand
// read a lane of row e = lane % 8 and chunk c = lane / 8 mod 4 starts at bank
// 4 (4 e + c) mod 64 with this line stride, and the quads of one pass hold
// distinct (e mod 4, c) pairs, so every pass touches 64 distinct banks (a
// 288-byte stride, with 72 e + 4 c, wraps two lanes of a pass onto one bank).
// Both addresses are one lane constant plus an immediate.
constexpr int kVtLine = 320;

// One block of 32 * WAVES query rows (query block qb of (sequence, head) hs),
// staged through the workgroup's LDS.
template <int D, bool kWithO, int WAVES>
__device__ __forceinline__ void fa_block(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int T_ctx,
    int Hq, int Hkv, float scale_log2, __bf16* __restrict__ o, float* __restrict__ lse, int hs, int qb,
    uint16_t* __restrict__ sK, char* __restrict__ sV, int w0, float* __restrict__ s_wl) {
    constexpr int NT = 64 * WAVES;          // threads
    constexpr int BM = 32 * WAVES;          // query rows per workgroup
    constexpr int CH = D / 8;               // 16-byte chunks per row
    constexpr int KS = D / 16;              // MFMA k-steps over the head dim
    constexpr int DB = D / 32;              // 32-wide output blocks over the head dim
    constexpr int LOADS = kBN * CH / NT;    // K chunks per thread per tile
    constexpr int KST = kKStride<D>;
    constexpr int TILE = kBN * KST;         // elements of one staged K tile
    constexpr int CH2 = D / 64;             // 64-wide halves of the head dim
    constexpr int VT_BYTES = 32 * CH2 * kVtLine;  // one staged V^T tile (padded lines)
    static_assert(!kWithO || WAVES == 8, "the V^T staging map assumes 8 waves");
    const int b = hs / Hq;
    const int h = hs % Hq;
    const int g = h / (Hq / Hkv);
    const int q0 = qb * BM;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int half = lane >> 5;
    // Waves w and w + 4 share a SIMD; giving them row groups w and 7 - w evens
    // out the causal work per SIMD, so the lone wave of a SIMD near the diagonal
    // has it to itself for longer.
    const int rgrp = WAVES == 8 && wave >= 4 ? 11 - wave : wave;
    const int qw0 = q0 + 32 * rgrp;
    const int qi = qw0 + (lane & 31);

    const size_t qbase = ((size_t)b * Hq + h) * T_ctx;
    const size_t kvbase = ((size_t)b * Hkv + g) * T_ctx;

    // Q^T operand: lane holds q[qi][16 kk + 8 half + 0..7] (loaded after the
    // first K / V tiles, which are needed first)
    bf16x8 qreg[KS];

    const int kv_end = min(T_ctx, q0 + BM);  // keys this workgroup needs
    const int ntiles = (kv_end + kBN - 1) / kBN;

    // K tiles are register-staged (global -> VGPR -> LDS, rows in lane order,
    // see kKStride).  Loads go through a buffer resource based at the tile's
    // first row and sized to the rows that exist: rows past T read as zeros
    // (a tile that starts past T reads nothing), and such keys sit only in
    // diagonal tiles, where they are masked, or in stages no QK^T reads.  (A
    // global_load_lds path would skip the VGPR hop, but the compiler then waits
    // for every outstanding load before any LDS read.)
    u32x4 pk[LOADS];
    // Row and chunk of the first 16-byte chunk this thread stages; its later
    // chunks are kRowStep rows further down.
    const int row0 = (int)(threadIdx.x / CH);
    const int col0 = 8 * (int)(threadIdx.x % CH);
    constexpr int kRowStep = NT / CH;
    const int goff0 = (row0 * D + col0) * 2;  // byte offset of chunk 0 inside a tile
    auto tile_rsrc = [&](const uint16_t* base, int n0) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base + (kvbase + (size_t)n0) * D), 0,
                                                 max(T_ctx - n0, 0) * D * 2, 0x00020000);
    };
    auto load_k_into = [&](int n0, u32x4 (&dst)[LOADS]) {
        const auto rk = tile_rsrc(k, n0);
#pragma unroll
        for (int i = 0; i < LOADS; ++i)
            dst[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, goff0 + i * kRowStep * D * 2, 0, 0));
    };
    auto store_k_part = [&](int buf, const u32x4 (&src)[LOADS], int i) {
        const int r = row0 + kRowStep * i, c = col0 / 8;
        *reinterpret_cast<u32x4*>(sK + buf * TILE + (32 * (r >> 5) + key_lane(r & 31)) * KST + 8 * c) = src[i];
    };
    auto store_k_from = [&](int buf, const u32x4 (&src)[LOADS]) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) store_k_part(buf, src, i);
    };
    auto load_k = [&](int n0) { load_k_into(n0, pk); };
    auto store_k = [&](int buf) { store_k_from(buf, pk); };
    // V tiles are register-staged, converted to fp16 and stored transposed
    // (V^T, see kVtLine): thread (bk, s, c_hi from the wave; c_lo, dw, half from
    // the lane) loads the 16-byte chunk c = 8 c_hi + c_lo of keys 2j and 2j+1,
    // j = 16 bk + 8 half + 4 s + dw, and writes the eight fp16 pairs
    // (V[2j][8c+e], V[2j+1][8c+e]) as dwords of V^T rows 8c+e.
    const int vw = wave;
    const bool v_active = 4 * CH2 >= WAVES || vw < 4 * CH2;  // D = 64 needs half of the waves
    const int v_chi = vw % CH2, v_s = (vw / CH2) & 1, v_bk = (vw / CH2 / 2) & 1;
    const int v_clo = lane & 7, v_dw = (lane >> 3) & 3, v_half = lane >> 5;
    const int v_j = 16 * v_bk + 8 * v_half + 4 * v_s + v_dw;
    const int goffv = (2 * v_j * D + 8 * (8 * v_chi + v_clo)) * 2;
    const int woffv = kVtLine * 8 * ((v_bk * 2 + v_s) * CH2 + v_chi) + 16 * (v_clo + 8 * v_half) + 4 * v_dw;
    u32x4 pv[kWithO ? 2 : 1];
    auto load_v = [&](int n0) {
        if constexpr (kWithO) {
            const auto rv = tile_rsrc(v, n0);
            if (v_active) {
                pv[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, goffv, 0, 0));
                pv[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, goffv + 2 * D, 0, 0));
            }
        }
    };

    auto store_v_part = [&](int buf, int w) {
        if constexpr (kWithO) {
            if (v_active) {
                char* dst = sV + buf * VT_BYTES + woffv;
                const f16x2 lo = {(_Float16)__uint_as_float(pv[0][w] << 16), (_Float16)__uint_as_float(pv[1][w] << 16)};
                const f16x2 hi = {(_Float16)__uint_as_float(pv[0][w] & 0xFFFF0000u),
                                  (_Float16)__uint_as_float(pv[1][w] & 0xFFFF0000u)};
                *reinterpret_cast<f16x2*>(dst + kVtLine * (2 * w)) = lo;
                *reinterpret_cast<f16x2*>(dst + kVtLine * (2 * w + 1)) = hi;
            }
        }
    };
    auto store_v = [&](int buf) {
#pragma unroll
        for (int w = 0; w < 4; ++w) store_v_part(buf, w);
    };

    // Softmax state of this lane's query, log2 domain.  m_ref is the reference
    // max the probabilities are taken against; it moves only when a tile's max
    // exceeds it by more than 8, so p <= 2^8 and the accumulators are rescaled
    // rarely (the result does not depend on m_ref).
    float m_ref = -INFINITY;
    float lsum = 0.0f;  // partial sum over this lane's half of the keys
    f32x16 oacc[kWithO ? DB : 1];
#pragma unroll
    for (int d = 0; d < (kWithO ? DB : 1); ++d) oacc[d] = f32x16{};

    // Per-lane LDS offset (elements) of the K operand: k-step kk of key block
    // bk is at koff + 16 kk + 32 bk KST.
    const int koff = (lane & 31) * KST + 8 * half;
    // V^T operand of head-dim block d, key block bk, key half s: the 16-byte
    // chunk (row 32 d + lane % 32, keys 32 bk + 16 half + 8 s + 0..7), at byte
    // voff + vt_imm(d, bk, s).
    const int voff = kVtLine * (lane & 7) + 16 * ((lane >> 3) & 3) + 128 * half;

    // S^T = K Q^T of the tile in stage `buf`, one 32-key block at a time; the
    // K operands are requested four k-steps at a time, each group before the
    // MFMAs that use it (fewer live registers while the softmax runs).
    auto qk = [&](int buf, f32x16 (&sacc)[2]) {
        const uint16_t* tk = sK + buf * TILE + koff;
        constexpr int G = KS < 4 ? KS : 4;
#pragma unroll
        for (int bk = 0; bk < 2; ++bk) {
            sacc[bk] = f32x16{};
#pragma unroll
            for (int k0 = 0; k0 < KS; k0 += G) {
                bf16x8 a[G];
#pragma unroll
                for (int kk = 0; kk < G; ++kk)
                    a[kk] = *reinterpret_cast<const bf16x8*>(tk + 16 * (k0 + kk) + 32 * bk * KST);
#pragma unroll
                for (int kk = 0; kk < G; ++kk)
                    sacc[bk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk], qreg[k0 + kk], sacc[bk], 0, 0, 0);
            }
        }
    };
    // Online softmax of one tile: returns the fp16 probabilities (PV operand)
    // and folds the fp32 row sum into lsum; rescales O when the reference max
    // moves.  Branch-free except the (rare, wave-uniform) rescale.
    auto softmax = [&](f32x16 (&sacc)[2], int n0, auto mask_tag, f16x8 (&pb)[2][2]) {
        constexpr bool kMask = decltype(mask_tag)::value;
        // key 32 bk + e of the lane's half lies past its query when 32 bk + e >
        // rel: the offsets are immediates, and rel is formed here, so no
        // per-key position is kept across the block
        int rel = qi - n0 - 16 * half;
        if constexpr (kMask) asm volatile("" : "+v"(rel));
        float tmax = -INFINITY;
#pragma unroll
        for (int bk = 0; bk < 2; ++bk) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                if constexpr (kMask) {
                    if (32 * bk + e > rel) sacc[bk][e] = -INFINITY;
                }
                tmax = fmaxf(tmax, sacc[bk][e]);
            }
        }
        const float tm = fmaxf(tmax, swap_halves(tmax)) * scale_log2;
        const float m_new = tm > m_ref + 8.0f ? tm : m_ref;
        const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);  // 1 unless the max moved
        const bool moved = m_new != m_ref;
        m_ref = m_new;
        float psum = 0.0f;
#pragma unroll
        for (int bk = 0; bk < 2; ++bk) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sacc[bk][e], scale_log2, -m_ref));
                psum += p;
                pb[bk][e >> 3][e & 7] = (_Float16)p;
            }
        }
        lsum = fmaf(lsum, alpha, psum);
        return moved;
    };

    // this wave's diagonal tile, the last one it needs (wave-uniform)
    const int t_last = __builtin_amdgcn_readfirstlane(min(qw0 / kBN, ntiles - 1));

    // O^T += V^T P^T of the tile in stage `buf`, one 32-wide block of the head
    // dim at a time (the order every accumulator takes its products in).
    auto pv_mma = [&](int buf, const f16x8 (&pb)[2][2]) {
        const char* tv = sV + buf * VT_BYTES + voff;
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
            for (int bk = 0; bk < 2; ++bk)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const f16x8 a = *reinterpret_cast<const f16x8*>(
                        tv + kVtLine * 8 * ((bk * 2 + s) * CH2 + (d >> 1)) + 64 * (d & 1));
                    oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[bk][s], oacc[d], 0, 0, 0);
                }
    };
    auto rescale = [&](bool moved, float alpha) {
        if constexpr (kWithO) {
            if (__ballot(moved)) {  // wave-uniform, rare
#pragma unroll
                for (int d = 0; d < DB; ++d)
#pragma unroll
                    for (int e = 0; e < 16; ++e) oacc[d][e] *= alpha;
            }
        }
    };

    // Steady-state tile t (0 < t < this wave's diagonal tile): the PV product of
    // tile t-1 (stage (t-1)&1, probabilities pbp) and the QK^T product of tile
    // t+1 (stage (t+1)&1, into sn) go to the matrix cores one MFMA per slot,
    // while the online softmax of tile t (sc, into pbn) is spread over the same
    // slots on the VALU, as are the staging writes of V(t) and K(t+2) into stage
    // t&1 and the loads of K(t+2) and V(t+1).  Scheduling barriers between the
    // slots and empty asm statements that pin values to their slot keep that
    // order; the arithmetic and its order are those of qk, softmax and pv_mma.
    auto step_a = [&](int t, f32x16 (&sc)[2], f32x16 (&sn)[2], const f16x8 (&pbp)[2][2], f16x8 (&pbn)[2][2]) {
        const int n0 = t * kBN;
        const int buf = t & 1;
        const uint16_t* tk = sK + (buf ^ 1) * TILE + koff;
        const char* tv = sV + (buf ^ 1) * VT_BYTES + voff;
        constexpr int NM = 2 * KS;             // MFMAs of one QK^T (and of one PV)
        constexpr int NPV = kWithO ? NM : 0;   // PV slots
        constexpr int NS = NPV + NM;           // slots
        constexpr int AHEAD = 4;               // operand reads in flight ahead of their MFMA
        constexpr int MS = 3;                  // slots that take the row max
        constexpr int ES = NS - MS;            // slots that take the exponentials
        constexpr int VS0 = 1;                 // slots VS0..VS0+3 write V(t); V(t+1) is loaded after
        constexpr int KS0 = NS - 1 - LOADS;    // slots that write K(t+2)
        u32x4 op[NS];
        auto read_op = [&](int r) {
            if (r < NPV) {
                const int bs = r / DB, d = r % DB, bk = bs >> 1, s = bs & 1;
                op[r] = *reinterpret_cast<const u32x4*>(tv + kVtLine * 8 * ((bk * 2 + s) * CH2 + (d >> 1)) + 64 * (d & 1));
            } else {
                const int j = r - NPV;
                op[r] = *reinterpret_cast<const u32x4*>(tk + 16 * (j % KS) + 32 * (j / KS) * KST);
            }
        };
        auto pin = [](auto& x) { asm volatile("" : "+v"(x)); };
        float tmax = -INFINITY, psum = 0.0f, alpha = 1.0f;
        bool moved = false;
        uint32_t pw[16];  // fp16 pairs of P(t)
        __builtin_amdgcn_sched_barrier(0);
        load_k(n0 + 2 * kBN);  // K(t+2); rows past the end read as zeros
#pragma unroll
        for (int r = 0; r < AHEAD; ++r) read_op(r);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            if (i + AHEAD < NS) read_op(i + AHEAD);
            if (i < NPV) {
                const int bs = i / DB, d = i % DB;
                oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, op[i]), pbp[bs >> 1][bs & 1],
                                                                 oacc[d], 0, 0, 0);
            } else {
                const int j = i - NPV;
                if (j % KS == 0) sn[j / KS] = f32x16{};
                sn[j / KS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, op[i]), qreg[j % KS],
                                                                     sn[j / KS], 0, 0, 0);
            }
            if (i < MS) {
#pragma unroll
                for (int e = 32 * i / MS; e < 32 * (i + 1) / MS; ++e) tmax = fmaxf(tmax, sc[e >> 4][e & 15]);
                if (i == MS - 1) {
                    const float tm = fmaxf(tmax, swap_halves(tmax)) * scale_log2;
                    const float m_new = tm > m_ref + 8.0f ? tm : m_ref;
                    alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
                    moved = m_new != m_ref;
                    m_ref = m_new;
                    pin(m_ref);
                }
            } else {
                const int jj = i - MS;
                const int e0 = 32 * jj / ES, e1 = 32 * (jj + 1) / ES;
#pragma unroll
                for (int e = e0; e < e1; ++e) {
                    float x = sc[e >> 4][e & 15];
                    pin(x);
                    sc[e >> 4][e & 15] = x;
                }
#pragma unroll
                for (int e = e0; e < e1; ++e) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(sc[e >> 4][e & 15], scale_log2, -m_ref));
                    psum += p;
                    sc[e >> 4][e & 15] = p;
                    if (e & 1) {
                        const f16x2 h = {(_Float16)sc[e >> 4][(e & 15) - 1], (_Float16)p};
                        pw[e >> 1] = __builtin_bit_cast(uint32_t, h);
                        pin(pw[e >> 1]);
                    }
                }
                pin(psum);
            }
            if constexpr (kWithO) {
                if (i >= VS0 && i < VS0 + 4) store_v_part(buf, i - VS0);  // V(t) -> stage t&1
                if (i == VS0 + 4) load_v(n0 + kBN);                       // V(t+1)
            }
            if (i >= KS0 && i < KS0 + LOADS) store_k_part(buf, pk, i - KS0);  // K(t+2) -> stage t&1
            __builtin_amdgcn_sched_barrier(0);
        }
        lsum = fmaf(lsum, alpha, psum);
#pragma unroll
        for (int bk = 0; bk < 2; ++bk)
#pragma unroll
            for (int hs2 = 0; hs2 < 2; ++hs2)
                pbn[bk][hs2] = __builtin_bit_cast(f16x8, u32x4{pw[8 * bk + 4 * hs2], pw[8 * bk + 4 * hs2 + 1],
                                                              pw[8 * bk + 4 * hs2 + 2], pw[8 * bk + 4 * hs2 + 3]});
        rescale(moved, alpha);
    };

    // Any other tile t, in plain order: PV(t-1), the staging of V(t) and the
    // load of V(t+1), then the softmax of tile t (with the QK^T of tile t+1
    // before the diagonal tile, masked on it), then the staging of K(t+2).
    // Tile ntiles exists only for the PV of the last tile.
    auto step_g = [&](int t, f32x16 (&sc)[2], f16x8 (&pb)[2][2]) {
        const int n0 = t * kBN;
        const int buf = t & 1;
        if (t + 2 < ntiles) load_k(n0 + 2 * kBN);
        if constexpr (kWithO) {
            if (t >= 1 && t - 1 <= t_last) pv_mma(buf ^ 1, pb);
            if (t < ntiles) store_v(buf);
            if (t + 1 < ntiles) load_v(n0 + kBN);
        }
        if (t <= t_last) {
            bool moved;
            const float m_old = m_ref;
            if (t < t_last) {
                f32x16 snext[2];
                qk(buf ^ 1, snext);
                moved = softmax(sc, n0, std::false_type{}, pb);
                sc[0] = snext[0];
                sc[1] = snext[1];
            } else {
                moved = softmax(sc, n0, std::true_type{}, pb);
            }
            rescale(moved, __builtin_amdgcn_exp2f(m_old - m_ref));
        }
        if (t + 2 < ntiles) store_k(buf);
    };

    // Software pipeline over the key tiles: tile t's softmax runs while the
    // matrix cores take tile t-1's PV and tile t+1's QK^T.  K is staged two
    // tiles ahead (K(t+2) written during tile t), V one tile ahead of its use
    // (V(t) written during tile t, read by PV(t) during tile t+1); one barrier
    // per tile.  The stage a write reuses was last read before the previous
    // barrier: K(t) by QK(t) during tile t-1, V(t-2) by PV(t-2) during tile t-1.
    {  // first two K tiles and the first V tile: all loads in flight at once
        u32x4 pk1[LOADS];
        load_k(0);
        load_v(0);  // V(0) stays in registers until tile 0 writes it
        if (ntiles > 1) load_k_into(kBN, pk1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            if (qi < T_ctx)
                qreg[kk] = *reinterpret_cast<const bf16x8*>(q + (qbase + qi) * D + 16 * kk + 8 * half);
            else
                qreg[kk] = bf16x8{};
        }
        __builtin_amdgcn_sched_barrier(0);
        store_k(0);
        if (ntiles > 1) store_k_from(1, pk1);
    }
    __syncthreads();
    f32x16 sacc[2], snext[2];
    f16x8 pb[2][2], pbn[2][2];
    qk(0, sacc);
    __syncthreads();  // every wave has read K(0) before tile 0 writes K(2) over it
    step_g(0, sacc, pb);
    __syncthreads();
    int t = 1;
    for (; t + 1 < t_last; t += 2) {
        step_a(t, sacc, snext, pb, pbn);
        __syncthreads();
        step_a(t + 1, snext, sacc, pbn, pb);
        __syncthreads();
    }
    if (t < t_last) {
        step_a(t, sacc, snext, pb, pbn);
        sacc[0] = snext[0];
        sacc[1] = snext[1];
#pragma unroll
        for (int bk = 0; bk < 2; ++bk)
#pragma unroll
            for (int hs2 = 0; hs2 < 2; ++hs2) pb[bk][hs2] = pbn[bk][hs2];
        __syncthreads();
        ++t;
    }
    for (; t <= ntiles; ++t) {
        step_g(t, sacc, pb);
        __syncthreads();
    }

    const float ltot = lsum + swap_halves(lsum);
    if (qi < T_ctx) {
        const float lse_i = (m_ref + __log2f(ltot)) * kLn2;
        if (half == 0) lse[qbase + qi] = lse_i;
        // observation rows of a fused score pass: the log2-domain lse the second
        // pass would derive from the stored value, bit for bit
        if (s_wl && half == 0 && qi >= w0) s_wl[qi - w0] = lse_i * wmass::kLog2e;
    }
    if constexpr (kWithO) {
        const float inv = 1.0f / ltot;
        if constexpr (D == 128) {
            // The wave's 32 rows of O go through its own 4 KB slice of the V^T
            // stages (free after the last tile: the next block writes them only
            // after its first barrier), 64 columns at a time, so that every
            // global store writes whole 128-byte half rows.  In the slice, row r
            // keeps its 16-byte chunk c at chunk c ^ ((r >> 1) & 7), which leaves
            // the lane-quad passes of the 16-byte reads free of bank conflicts.
            char* so = sV + wave * (32 * 128);
            // lane index formed here, so the slice and store addresses are
            // computed in the epilogue instead of being kept (spilled) across
            // the tile loop
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const int r = ln & 31;
#pragma unroll
            for (int R = 0; R < 2; ++R) {
#pragma unroll
                for (int dd = 0; dd < 2; ++dd) {
#pragma unroll
                    for (int a4 = 0; a4 < 4; ++a4) {
                        bf16x4 w;
#pragma unroll
                        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(oacc[2 * R + dd][4 * a4 + e] * inv);
                        *reinterpret_cast<bf16x4*>(so + r * 128 + 16 * ((4 * dd + a4) ^ ((r >> 1) & 7)) + 8 * half) = w;
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = (ln >> 3) + 8 * i, c = ln & 7;
                    const u32x4 val = *reinterpret_cast<const u32x4*>(so + rr * 128 + 16 * (c ^ ((rr >> 1) & 7)));
                    if (qw0 + rr < T_ctx)
                        *reinterpret_cast<u32x4*>(o + (qbase + qw0 + rr) * D + 64 * R + 8 * c) = val;
                }
            }
        } else if (qi < T_ctx) {
#pragma unroll
            for (int d = 0; d < DB; ++d) {
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    bf16x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = (__bf16)(oacc[d][4 * a4 + e] * inv);
                    *reinterpret_cast<bf16x4*>(o + (qbase + qi) * D + 32 * d + 8 * a4 + 4 * half) = w;
                }
            }
        }
    }
}

// Window scores of (sequence, head) hs from inside pass 1: the W <= 32 rows
// T-W..T-1 (Q operand from L2, lse from LDS) against every key; the waves of
// the workgroup take contiguous runs of 32-key blocks, K blocks come through
// two register sets (the next one loading while the current one is reduced).
// One query head per KV head, so the scores row is the head's own.
template <int D, int WAVES>
__device__ __forceinline__ void window_tail(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, int T_ctx,
                                            int hs, int W, float scale_log2, const float* __restrict__ s_wl,
                                            float* __restrict__ scores) {
    constexpr int KS = D / 16;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int half = lane >> 5;
    const size_t base = (size_t)hs * T_ctx;
    const int w0 = T_ctx - W;
    const int nkb = (T_ctx + 31) / 32;
    const int per = (nkb + WAVES - 1) / WAVES;
    const int kb0 = wave * per;
    const int nb = min(per, nkb - kb0);
    if (nb <= 0) return;
    bf16x8 qa[KS];
    float l2[16];
    wmass::load_qrows<D>(q, base, w0, W, 0, lane, qa);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int m = wmass::acc_row(e, lane);
        l2[e] = m < W ? s_wl[m] : INFINITY;
    }
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(k + base * D), 0, T_ctx * D * 2, 0x00020000);
    auto emit = [&](int i, float a) {
        a += swap_halves(a);
        const int j = (kb0 + i) * 32 + (lane & 31);
        if (half == 0 && j < T_ctx) scores[base + j] = a;
    };
    bf16x8 ka[KS], kb[KS];
    wmass::load_kblock<D>(rk, kb0 * 32, lane, ka);
    for (int i = 0; i < nb; i += 2) {
        if (i + 1 < nb) wmass::load_kblock<D>(rk, (kb0 + i + 1) * 32, lane, kb);
        emit(i, wmass::block_mass<D>(qa, ka, l2, scale_log2, w0, (kb0 + i) * 32, lane));
        if (i + 2 < nb) wmass::load_kblock<D>(rk, (kb0 + i + 2) * 32, lane, ka);
        if (i + 1 < nb) emit(i + 1, wmass::block_mass<D>(qa, kb, l2, scale_log2, w0, (kb0 + i + 1) * 32, lane));
    }
}

// Persistent workgroups, one per CU, dispatched round-robin over the XCDs
// (workgroup L on XCD L % 8).  Each XCD owns a contiguous run of (sequence,
// head) pairs, so the K/V prefix a head's query blocks re-read stays in that
// XCD's L2.  Within an XCD the query blocks of each head are taken in pairs
// (qb, nqb - 1 - qb), which cost the same, and the pairs are dealt round-robin
// to the XCD's workgroups: equal work per workgroup, and no re-dispatch gaps
// between blocks (a block's output stores drain while the next one loads).
// With fused window scores (W > 0) each head's pairs are rotated by the round
// they run in, so the pair that carries a score pass lands on a different
// workgroup in every round (one per workgroup when heads and pairs tile the
// XCD evenly) and score passes overlap other workgroups' attention.
template <int D, bool kWithO, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void fa_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int B_,
    int T_ctx, int Hq, int Hkv, int nqb, float scale_log2, __bf16* __restrict__ o, float* __restrict__ lse,
    int W, float* __restrict__ scores) {
    constexpr int TILE = kBN * kKStride<D>;
    constexpr int VT_BYTES = 32 * (D / 64) * kVtLine;
    // two LDS stages: tile t is read from one while tile t+1 is written to the other
    __shared__ __attribute__((aligned(16))) uint16_t sK[2 * TILE];
    __shared__ __attribute__((aligned(16))) char sV[kWithO ? 2 * VT_BYTES : 16];
    __shared__ float s_wl[32];  // log2-domain lse of the observation rows (fused scores)

    const int heads = B_ * Hq;
    const int per = (heads + kXcds - 1) / kXcds;
    const int xcd = blockIdx.x % kXcds;
    const int slot = blockIdx.x / kXcds;
    const int nslots = gridDim.x / kXcds;
    const int h0 = xcd * per;
    const int nh = max(0, min(heads, h0 + per) - h0);
    const int pairs = (nqb + 1) / 2;  // per head
    // one call site: (pair p, second) walks the long then the short block of each pair
    int p = slot;
    bool second = false;
    while (p < nh * pairs) {
        const int hs = h0 + p / pairs;
        // the rotation depends on the head alone, so it permutes the head's pairs
        const int j = W == 0 ? p % pairs : (p % pairs + (p / pairs) * pairs / nslots) % pairs;
        const int qb = second ? j : nqb - 1 - j;
        const bool tail = W > 0 && qb == nqb - 1;
        fa_block<D, kWithO, WAVES>(q, k, v, T_ctx, Hq, Hkv, scale_log2, o, lse, hs, qb, sK, sV, T_ctx - W,
                                   tail ? s_wl : nullptr);
        if (tail) {
            __syncthreads();  // the observation rows' lse are in s_wl
            window_tail<D, WAVES>(q, k, T_ctx, hs, W, scale_log2, s_wl, scores);
            __syncthreads();  // s_wl and the waves are free for the next block
        }
        if (!second && j != nqb - 1 - j) {
            second = true;
        } else {
            second = false;
            p += nslots;
        }
    }
}

int cu_count() { return device_cu_count(); }

template <int D, bool kWithO>
hipError_t launch_fa(const void* q, const void* k, const void* v, int B, int T_ctx, int Hq, int Hkv,
                     float sm_scale, void* o, float* lse, int W, float* scores, hipStream_t stream) {
    constexpr int WAVES = kFaWaves;
    const int nqb = (T_ctx + 32 * WAVES - 1) / (32 * WAVES);
    const int grid = max(kXcds, cu_count() / kXcds * kXcds);
    hipLaunchKernelGGL((fa_fwd_kernel<D, kWithO, WAVES>), dim3(grid), dim3(64 * WAVES), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), B, T_ctx, Hq, Hkv, nqb, sm_scale * kLog2e,
                       static_cast<__bf16*>(o), lse, W, scores);
    return hipGetLastError();
}

}  // namespace

int device_cu_count() {
    static int n = 0;
    if (n == 0) {
        int dev = 0, c = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0)
            n = c;
        else
            n = 256;
    }
    return n;
}

// One score pass per head runs on the workgroup that finishes the head's last
// query block, its 8 waves walking the head's keys; with fewer heads than
// workgroups those few long passes would trail the kernel, and the stand-alone
// pass, spread over the whole GPU, is faster.
bool prefill_fuses_scores(int B, int T_ctx, int Hq, int Hkv, int window) {
    constexpr int BM = 32 * kFaWaves;
    const int last_rows = T_ctx - (T_ctx - 1) / BM * BM;  // rows of the last query block
    return Hq == Hkv && window >= 1 && window <= 32 && window <= last_rows &&
           (long long)B * Hq >= cu_count();
}

hipError_t launch_prefill(const void* q, const void* k, const void* v, int B, int T_ctx, int Hq, int Hkv,
                          int D, float sm_scale, void* o, float* lse, int window, float* scores,
                          hipStream_t stream) {
    if (window != 0 && (!scores || !prefill_fuses_scores(B, T_ctx, Hq, Hkv, window))) return hipErrorInvalidValue;
    if (D == 128) {
        if (o) return launch_fa<128, true>(q, k, v, B, T_ctx, Hq, Hkv, sm_scale, o, lse, window, scores, stream);
        return launch_fa<128, false>(q, k, v, B, T_ctx, Hq, Hkv, sm_scale, o, lse, window, scores, stream);
    }
    if (o) return launch_fa<64, true>(q, k, v, B, T_ctx, Hq, Hkv, sm_scale, o, lse, window, scores, stream);
    return launch_fa<64, false>(q, k, v, B, T_ctx, Hq, Hkv, sm_scale, o, lse, window, scores, stream);
}

}  // namespace minikv
