// C ABI of the library: argument validation (before any HIP call), launch.
#include <math.h>

#include "minikv.h"
#include "kernels.h"

namespace {

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int status_of(hipError_t e) { return e == hipSuccess ? MINIKV_OK : MINIKV_ERR_LAUNCH; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

float resolve_scale(float sm_scale, int D) { return sm_scale > 0.0f ? sm_scale : 1.0f / sqrtf((float)D); }

bool supported_d(int D) { return D == 64 || D == 128; }

// The kernels address one (sequence, head) slice of K / V (T rows of D
// elements) through a 32-bit buffer range, so its bytes must stay below 2 GiB.
bool slice_fits(int T, int D, int elem_bytes) { return (long long)T * D * elem_bytes <= 0x7fffffffLL; }

}  // namespace

extern "C" {

#ifndef MINIKV_BUILD_ID
#define MINIKV_BUILD_ID "sha256:unknown"
#endif
const char* minikv_build_id(void) { return MINIKV_BUILD_ID; }

int minikv_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    if (!src || !sink) return MINIKV_ERR_NULL;
    if (bytes == 0 || bytes % 16) return MINIKV_ERR_SHAPE;
    if (misaligned(src) || misaligned(sink)) return MINIKV_ERR_ALIGN;
    return status_of(minikv::launch_read_probe(src, bytes, sink, MINIKV_READ_PROBE_SINK_WORDS, as_stream(stream)));
}

const char* minikv_status_string(int status) {
    switch (status) {
        case MINIKV_OK: return "ok";
        case MINIKV_ERR_NULL: return "a required pointer is NULL";
        case MINIKV_ERR_SHAPE: return "inconsistent or out-of-range sizes";
        case MINIKV_ERR_UNSUPPORTED: return "unsupported configuration";
        case MINIKV_ERR_ALIGN: return "pointer not 16-byte aligned";
        case MINIKV_ERR_WORKSPACE: return "workspace missing or too small";
        case MINIKV_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

size_t minikv_packed_bytes(int B, int Hkv, int n_keep, int D) {
    if (B < 1 || Hkv < 1 || n_keep < 1 || D < 32 || D % 32) return 0;
    const size_t n = (size_t)n_keep;
    const size_t groups = (n + MINIKV_GROUP - 1) / MINIKV_GROUP;
    const size_t per = n * D / 4 + groups * D * 4 + groups * MINIKV_GROUP * D / 4 + n * (D / MINIKV_GROUP) * 4;
    return (size_t)B * Hkv * per;
}

size_t minikv_decode_ws_bytes(int B, int Hq, int Hkv, int n_keep, int D) {
    if (B < 1 || Hq < 1 || Hkv < 1 || n_keep < 1 || Hq % Hkv || !supported_d(D)) return 0;
    return minikv::decode_ws_bytes(B, Hq, D, minikv::decode_plan(B, Hq, Hkv, n_keep, D));
}

int minikv_keep_count(int T, int pct_milli) {
    if (T < 1 || pct_milli <= 0 || pct_milli > 100000) return MINIKV_ERR_SHAPE;
    const long long n = (long long)pct_milli * T / 100000;
    return (int)(n < 1 ? 1 : n);
}

int minikv_pyramid_keep(int T, int n_layers, int layer, int first_pct, int last_pct) {
    if (T < 1 || n_layers < 1 || layer < 0 || layer >= n_layers || first_pct <= 0 || first_pct > 100 ||
        last_pct <= 0 || last_pct > 100)
        return MINIKV_ERR_SHAPE;
    long long n;
    if (n_layers == 1) {
        n = (long long)first_pct * T / 100;
    } else {
        const long long L1 = n_layers - 1;
        n = ((long long)first_pct * L1 + (long long)(last_pct - first_pct) * layer) * T / (100 * L1);
    }
    return (int)(n < 1 ? 1 : n);
}

int minikv_split_heavy_recent(int n_keep, int* n_heavy, int* n_recent) {
    if (!n_heavy || !n_recent) return MINIKV_ERR_NULL;
    if (n_keep < 1) return MINIKV_ERR_SHAPE;
    *n_recent = n_keep / 5;
    *n_heavy = n_keep - *n_recent;
    return MINIKV_OK;
}

namespace {
int check_prefill_args(const void* q, const void* k, const void* v, int B, int T, int Hq, int Hkv, int D) {
    if (!q || !k || !v) return MINIKV_ERR_NULL;
    if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv) return MINIKV_ERR_SHAPE;
    if (!supported_d(D) || !slice_fits(T, D, 2)) return MINIKV_ERR_UNSUPPORTED;
    if (misaligned(q) || misaligned(k) || misaligned(v)) return MINIKV_ERR_ALIGN;
    return MINIKV_OK;
}
}  // namespace

int minikv_prefill_attn(const void* q, const void* k, const void* v, int B, int T, int Hq, int Hkv, int D,
                        float sm_scale, void* o, float* lse, void* stream) {
    if (!lse) return MINIKV_ERR_NULL;
    const int st = check_prefill_args(q, k, v, B, T, Hq, Hkv, D);
    if (st != MINIKV_OK) return st;
    if (misaligned(lse) || (o && misaligned(o))) return MINIKV_ERR_ALIGN;
    return status_of(minikv::launch_prefill(q, k, v, B, T, Hq, Hkv, D, resolve_scale(sm_scale, D), o, lse, 0,
                                            nullptr, as_stream(stream)));
}

int minikv_window_scores(const void* q, const void* k, const float* lse, int B, int T, int Hq, int Hkv, int D,
                         int window, float sm_scale, float* scores, void* stream) {
    if (!lse || !scores) return MINIKV_ERR_NULL;
    const int st = check_prefill_args(q, k, k, B, T, Hq, Hkv, D);
    if (st != MINIKV_OK) return st;
    if (window < 1 || window > T) return MINIKV_ERR_SHAPE;
    if (misaligned(lse) || misaligned(scores)) return MINIKV_ERR_ALIGN;
    return status_of(minikv::launch_window_scores(q, k, lse, B, T, Hq, Hkv, D, window,
                                                  resolve_scale(sm_scale, D), scores, as_stream(stream)));
}

int minikv_prefill_attn_scores(const void* q, const void* k, const void* v, int B, int T, int Hq, int Hkv,
                               int D, int window, float sm_scale, void* o, float* lse, float* scores,
                               void* stream) {
    if (!lse || !scores) return MINIKV_ERR_NULL;
    int st = check_prefill_args(q, k, v, B, T, Hq, Hkv, D);
    if (st != MINIKV_OK) return st;
    if (window < 1 || window > T) return MINIKV_ERR_SHAPE;
    if (misaligned(lse) || misaligned(scores) || (o && misaligned(o))) return MINIKV_ERR_ALIGN;
    if (minikv::prefill_fuses_scores(B, T, Hq, Hkv, window))  // one launch: scores from inside pass 1
        return status_of(minikv::launch_prefill(q, k, v, B, T, Hq, Hkv, D, resolve_scale(sm_scale, D), o, lse,
                                                window, scores, as_stream(stream)));
    st = minikv_prefill_attn(q, k, v, B, T, Hq, Hkv, D, sm_scale, o, lse, stream);
    if (st != MINIKV_OK) return st;
    return minikv_window_scores(q, k, lse, B, T, Hq, Hkv, D, window, sm_scale, scores, stream);
}

int minikv_prefill_fuses_scores(int B, int T, int Hq, int Hkv, int window) {
    if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || window < 1 || window > T) return 0;
    return minikv::prefill_fuses_scores(B, T, Hq, Hkv, window) ? 1 : 0;
}

size_t minikv_select_ws_bytes(int B, int Hkv, int T) {
    // one workgroup per row keeps the row's keys (registers, or L2 re-reads past
    // 32 per thread) and its radix histograms (LDS) on chip: nothing in HBM
    (void)B;
    (void)Hkv;
    (void)T;
    return 0;
}

int minikv_select_topk(const float* scores, int B, int Hkv, int T, int n_heavy, int n_recent, int32_t* idx,
                       void* ws, size_t ws_bytes, void* stream) {
    if (!scores || !idx) return MINIKV_ERR_NULL;
    if (B < 1 || Hkv < 1 || T < 1 || n_heavy < 0 || n_recent < 0 || n_heavy + n_recent < 1 ||
        n_heavy + n_recent > T)
        return MINIKV_ERR_SHAPE;
    if (T - n_recent > 65536) return MINIKV_ERR_UNSUPPORTED;
    if (misaligned(scores) || misaligned(idx) || (ws && misaligned(ws))) return MINIKV_ERR_ALIGN;
    const size_t need = minikv_select_ws_bytes(B, Hkv, T);
    if (need > 0 && (!ws || ws_bytes < need)) return MINIKV_ERR_WORKSPACE;
    return status_of(minikv::launch_select_topk(scores, B, Hkv, T, n_heavy, n_recent, idx, as_stream(stream)));
}

int minikv_quant_pack(const void* k, const void* v, int in_dtype, const int32_t* idx, int B, int Hkv, int T,
                      int D, int n_keep, const minikv_packed_t* out, void* stream) {
    if (!k || !v || !out || !out->k_codes || !out->k_sz || !out->v_codes || !out->v_sz) return MINIKV_ERR_NULL;
    if (B < 1 || Hkv < 1 || T < 1 || n_keep < 1 || n_keep > T) return MINIKV_ERR_SHAPE;
    if (out->B != B || out->Hkv != Hkv || out->n_keep != n_keep || out->D != D) return MINIKV_ERR_SHAPE;
    if (!idx && n_keep != T) return MINIKV_ERR_SHAPE;
    if (!supported_d(D) || out->group != MINIKV_GROUP) return MINIKV_ERR_UNSUPPORTED;
    if (in_dtype != MINIKV_F32 && in_dtype != MINIKV_BF16) return MINIKV_ERR_UNSUPPORTED;
    if (!slice_fits(T, D, in_dtype == MINIKV_BF16 ? 2 : 4)) return MINIKV_ERR_UNSUPPORTED;
    if (misaligned(k) || misaligned(v) || (idx && misaligned(idx)) || misaligned(out->k_codes) ||
        misaligned(out->k_sz) || misaligned(out->v_codes) || misaligned(out->v_sz))
        return MINIKV_ERR_ALIGN;
    return status_of(minikv::launch_quant_pack(k, v, in_dtype == MINIKV_BF16, idx, B, Hkv, T, D, n_keep,
                                               out->k_codes, out->k_sz, out->v_codes, out->v_sz,
                                               as_stream(stream)));
}

int minikv_decode_attn(const void* q, const minikv_packed_t* cache, int Hq, float sm_scale, void* out, void* ws,
                       size_t ws_bytes, void* stream) {
    if (!q || !cache || !out || !cache->k_codes || !cache->k_sz || !cache->v_codes || !cache->v_sz)
        return MINIKV_ERR_NULL;
    const int B = cache->B, Hkv = cache->Hkv, n = cache->n_keep, D = cache->D;
    if (B < 1 || Hkv < 1 || n < 1 || Hq < 1 || Hq % Hkv) return MINIKV_ERR_SHAPE;
    if (!supported_d(D) || cache->group != MINIKV_GROUP) return MINIKV_ERR_UNSUPPORTED;
    const int R = Hq / Hkv;
    if (R != 1 && R != 2 && R != 4) return MINIKV_ERR_UNSUPPORTED;
    if (misaligned(q) || misaligned(out) || misaligned(cache->k_codes) || misaligned(cache->k_sz) ||
        misaligned(cache->v_codes) || misaligned(cache->v_sz) || (ws && misaligned(ws)))
        return MINIKV_ERR_ALIGN;
    const minikv::DecodePlan plan = minikv::decode_plan(B, Hq, Hkv, n, D);
    if (!ws || ws_bytes < minikv::decode_ws_bytes(B, Hq, D, plan)) return MINIKV_ERR_WORKSPACE;
    return status_of(minikv::launch_decode(q, cache->k_codes, cache->k_sz, cache->v_codes, cache->v_sz, B, Hq,
                                           Hkv, n, D, resolve_scale(sm_scale, D), out, ws, plan,
                                           as_stream(stream)));
}

int minikv_decode_attn_noalloc(const void* q, const minikv_packed_t* cache, int Hq, float sm_scale, void* out,
                               void* stream) {
    static_assert(minikv::kDecodeScratchBytes == MINIKV_DECODE_SCRATCH_BYTES, "scratch size");
    static_assert(minikv::kTicketBytes == MINIKV_DECODE_TICKET_BYTES, "ticket area");
    if (!q || !cache || !out || !cache->k_codes || !cache->k_sz || !cache->v_codes || !cache->v_sz)
        return MINIKV_ERR_NULL;
    const int B = cache->B, Hkv = cache->Hkv, n = cache->n_keep, D = cache->D;
    if (B < 1 || Hkv < 1 || n < 1 || Hq < 1 || Hq % Hkv) return MINIKV_ERR_SHAPE;
    if (!supported_d(D) || cache->group != MINIKV_GROUP) return MINIKV_ERR_UNSUPPORTED;
    const int R = Hq / Hkv;
    if (R != 1 && R != 2 && R != 4) return MINIKV_ERR_UNSUPPORTED;
    if (misaligned(q) || misaligned(out) || misaligned(cache->k_codes) || misaligned(cache->k_sz) ||
        misaligned(cache->v_codes) || misaligned(cache->v_sz))
        return MINIKV_ERR_ALIGN;
    const minikv::DecodePlan plan = minikv::decode_plan(B, Hq, Hkv, n, D);
    // one token range per KV head writes the output directly: no scratch used
    void* ws = nullptr;
    if (plan.splits > 1) {
        if (minikv::decode_ws_bytes(B, Hq, D, plan) > minikv::kDecodeScratchBytes) return MINIKV_ERR_WORKSPACE;
        ws = minikv::decode_scratch();
        if (!ws) return MINIKV_ERR_LAUNCH;
    }
    return status_of(minikv::launch_decode(q, cache->k_codes, cache->k_sz, cache->v_codes, cache->v_sz, B, Hq,
                                           Hkv, n, D, resolve_scale(sm_scale, D), out, ws, plan,
                                           as_stream(stream)));
}

int minikv_stream_pack(const void* k, const void* v, int in_dtype, const int32_t* idx, int idx_stride, int B,
                       int Hkv, int T, int D, int n, int cap, int tok0, uint8_t* k_codes, uint32_t* k_sz,
                       uint8_t* v_codes, uint32_t* v_sz, void* stream) {
    if (!k || !v || !k_codes || !k_sz || !v_codes || !v_sz) return MINIKV_ERR_NULL;
    if (B < 1 || Hkv < 1 || T < 1 || n < 1 || cap < 1 || tok0 < 0) return MINIKV_ERR_SHAPE;
    if (n % MINIKV_GROUP || tok0 % MINIKV_GROUP || cap % MINIKV_GROUP || tok0 + n > cap) return MINIKV_ERR_SHAPE;
    if (idx ? idx_stride < n : n > T) return MINIKV_ERR_SHAPE;
    if (!supported_d(D)) return MINIKV_ERR_UNSUPPORTED;
    if (in_dtype != MINIKV_F32 && in_dtype != MINIKV_BF16) return MINIKV_ERR_UNSUPPORTED;
    if (!slice_fits(T, D, in_dtype == MINIKV_BF16 ? 2 : 4)) return MINIKV_ERR_UNSUPPORTED;
    if (misaligned(k) || misaligned(v) || misaligned(k_codes) || misaligned(k_sz) || misaligned(v_codes) ||
        misaligned(v_sz))
        return MINIKV_ERR_ALIGN;
    return status_of(minikv::launch_stream_pack(k, v, in_dtype == MINIKV_BF16, idx, idx ? idx_stride : n, B, Hkv, T,
                                                D, n, cap, tok0, k_codes, k_sz, v_codes, v_sz, as_stream(stream)));
}

int minikv_stream_append(const void* k, const void* v, const int32_t* idx, int idx_stride, int B, int Hkv, int T,
                         int D, int n, int slot, void* k_res, void* v_res, void* stream) {
    if (!k || !v || !k_res || !v_res) return MINIKV_ERR_NULL;
    if (B < 1 || Hkv < 1 || T < 1 || n < 1 || slot < 0 || slot + n > MINIKV_GROUP) return MINIKV_ERR_SHAPE;
    if (idx ? idx_stride < n : n > T) return MINIKV_ERR_SHAPE;
    if (!supported_d(D) || !slice_fits(T, D, 2)) return MINIKV_ERR_UNSUPPORTED;
    if (misaligned(k) || misaligned(v) || misaligned(k_res) || misaligned(v_res)) return MINIKV_ERR_ALIGN;
    return status_of(minikv::launch_stream_append(k, v, idx, idx ? idx_stride : n, B, Hkv, T, D, n, slot, k_res,
                                                  v_res, as_stream(stream)));
}

int minikv_stream_init(const void* k, const void* v, const int32_t* idx, int B, int Hkv, int T, int D, int n_keep,
                       int cap, uint8_t* k_codes, uint32_t* k_sz, uint8_t* v_codes, uint32_t* v_sz, void* k_res,
                       void* v_res, int* n_packed, int* n_res, void* stream) {
    if (!k || !v || !idx || !k_codes || !k_sz || !v_codes || !v_sz || !k_res || !v_res || !n_packed || !n_res)
        return MINIKV_ERR_NULL;
    if (B < 1 || Hkv < 1 || T < 1 || n_keep < 1 || n_keep > T || cap < MINIKV_GROUP || cap % MINIKV_GROUP)
        return MINIKV_ERR_SHAPE;
    // whole 32-token groups are packed; the rest (at most 31) wait in the window
    const int pk = MINIKV_GROUP * (n_keep / MINIKV_GROUP), rest = n_keep - pk;
    if (pk > cap) return MINIKV_ERR_SHAPE;
    if (!supported_d(D) || !slice_fits(T, D, 2)) return MINIKV_ERR_UNSUPPORTED;
    if (misaligned(k) || misaligned(v) || misaligned(idx) || misaligned(k_codes) || misaligned(k_sz) ||
        misaligned(v_codes) || misaligned(v_sz) || misaligned(k_res) || misaligned(v_res))
        return MINIKV_ERR_ALIGN;
    const hipStream_t st = as_stream(stream);
    if (pk > 0) {
        const int e = status_of(minikv::launch_stream_pack(k, v, true, idx, n_keep, B, Hkv, T, D, pk, cap, 0,
                                                           k_codes, k_sz, v_codes, v_sz, st));
        if (e != MINIKV_OK) return e;
    }
    if (rest > 0) {
        const int e = status_of(minikv::launch_stream_append(k, v, idx + pk, n_keep, B, Hkv, T, D, rest, 0, k_res,
                                                             v_res, st));
        if (e != MINIKV_OK) return e;
    }
    *n_packed = pk;
    *n_res = rest;
    return MINIKV_OK;
}

int minikv_stream_append_token(const void* k_new, const void* v_new, int B, int Hkv, int D, int cap, int* n_packed,
                               int* n_res, uint8_t* k_codes, uint32_t* k_sz, uint8_t* v_codes, uint32_t* v_sz,
                               void* k_res, void* v_res, void* stream) {
    if (!k_new || !v_new || !n_packed || !n_res || !k_codes || !k_sz || !v_codes || !v_sz || !k_res || !v_res)
        return MINIKV_ERR_NULL;
    if (B < 1 || Hkv < 1 || cap < MINIKV_GROUP || cap % MINIKV_GROUP) return MINIKV_ERR_SHAPE;
    const int np = *n_packed, nr = *n_res;
    if (np < 0 || np % MINIKV_GROUP || np > cap || nr < 0 || nr >= MINIKV_GROUP) return MINIKV_ERR_SHAPE;
    // this token fills the window: it is packed as the next group, which must fit
    const bool flush = nr + 1 == MINIKV_GROUP;
    if (flush && np + MINIKV_GROUP > cap) return MINIKV_ERR_SHAPE;
    if (!supported_d(D)) return MINIKV_ERR_UNSUPPORTED;
    if (misaligned(k_new) || misaligned(v_new) || misaligned(k_codes) || misaligned(k_sz) || misaligned(v_codes) ||
        misaligned(v_sz) || misaligned(k_res) || misaligned(v_res))
        return MINIKV_ERR_ALIGN;
    const hipStream_t st = as_stream(stream);
    int e = status_of(minikv::launch_stream_append(k_new, v_new, nullptr, 1, B, Hkv, 1, D, 1, nr, k_res, v_res, st));
    if (e != MINIKV_OK) return e;
    if (flush) {
        e = status_of(minikv::launch_stream_pack(k_res, v_res, true, nullptr, MINIKV_GROUP, B, Hkv, MINIKV_GROUP, D,
                                                 MINIKV_GROUP, cap, np, k_codes, k_sz, v_codes, v_sz, st));
        if (e != MINIKV_OK) return e;
        *n_packed = np + MINIKV_GROUP;
        *n_res = 0;
    } else {
        *n_res = nr + 1;
    }
    return MINIKV_OK;
}

size_t minikv_stream_decode_ws_bytes(int B, int Hq, int Hkv, int n_packed, int n_res, int D) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || n_packed < 0 || n_packed % MINIKV_GROUP || n_res < 0 ||
        n_res >= MINIKV_GROUP || n_packed + n_res < 1 || !supported_d(D))
        return 0;
    const minikv::DecodePlan plan = minikv::decode_plan(B, Hq, Hkv, n_packed > 0 ? n_packed : 1, D);
    const size_t b = minikv::stream_decode_ws_bytes(B, Hq, D, n_packed, n_res, plan);
    return b ? b : 16;
}

int minikv_stream_decode(const void* q, int B, int Hq, int Hkv, int D, int cap, int n_packed,
                         const uint8_t* k_codes, const uint32_t* k_sz, const uint8_t* v_codes,
                         const uint32_t* v_sz, const void* k_res, const void* v_res, int n_res, float sm_scale,
                         void* out, void* ws, size_t ws_bytes, void* stream) {
    if (!q || !out) return MINIKV_ERR_NULL;
    if (n_packed > 0 && (!k_codes || !k_sz || !v_codes || !v_sz)) return MINIKV_ERR_NULL;
    if (n_res > 0 && (!k_res || !v_res)) return MINIKV_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || cap < 0 || cap % MINIKV_GROUP) return MINIKV_ERR_SHAPE;
    if (n_packed < 0 || n_packed % MINIKV_GROUP || n_packed > cap || n_res < 0 || n_res >= MINIKV_GROUP ||
        n_packed + n_res < 1)
        return MINIKV_ERR_SHAPE;
    if (!supported_d(D)) return MINIKV_ERR_UNSUPPORTED;
    const int R = Hq / Hkv;
    if (R != 1 && R != 2 && R != 4) return MINIKV_ERR_UNSUPPORTED;
    if (misaligned(q) || misaligned(out) || (ws && misaligned(ws)) ||
        (n_packed > 0 && (misaligned(k_codes) || misaligned(k_sz) || misaligned(v_codes) || misaligned(v_sz))) ||
        (n_res > 0 && (misaligned(k_res) || misaligned(v_res))))
        return MINIKV_ERR_ALIGN;
    const minikv::DecodePlan plan = minikv::decode_plan(B, Hq, Hkv, n_packed > 0 ? n_packed : 1, D);
    const size_t need = minikv::stream_decode_ws_bytes(B, Hq, D, n_packed, n_res, plan);
    if (need > 0 && (!ws || ws_bytes < need)) return MINIKV_ERR_WORKSPACE;
    return status_of(minikv::launch_stream_decode(q, k_codes, k_sz, v_codes, v_sz, B, Hq, Hkv, D, cap, n_packed,
                                                  k_res, v_res, n_res, resolve_scale(sm_scale, D), out, ws, plan,
                                                  as_stream(stream)));
}

int minikv_stream_set_counts(int32_t* counts, int n_packed, int n_res, int cap, void* stream) {
    if (!counts) return MINIKV_ERR_NULL;
    if (cap < MINIKV_GROUP || cap % MINIKV_GROUP || n_packed < 0 || n_packed % MINIKV_GROUP || n_packed > cap ||
        n_res < 0 || n_res >= MINIKV_GROUP)
        return MINIKV_ERR_SHAPE;
    if (misaligned(counts)) return MINIKV_ERR_ALIGN;
    return status_of(minikv::launch_stream_set_counts(counts, n_packed, n_res, as_stream(stream)));
}

int minikv_stream_step_append(const void* k_new, const void* v_new, int B, int Hkv, int D, int cap,
                              int32_t* counts, uint8_t* k_codes, uint32_t* k_sz, uint8_t* v_codes, uint32_t* v_sz,
                              void* k_res, void* v_res, void* stream) {
    if (!k_new || !v_new || !counts || !k_codes || !k_sz || !v_codes || !v_sz || !k_res || !v_res)
        return MINIKV_ERR_NULL;
    if (B < 1 || Hkv < 1 || cap < MINIKV_GROUP || cap % MINIKV_GROUP) return MINIKV_ERR_SHAPE;
    if (!supported_d(D)) return MINIKV_ERR_UNSUPPORTED;
    if (misaligned(k_new) || misaligned(v_new) || misaligned(counts) || misaligned(k_codes) || misaligned(k_sz) ||
        misaligned(v_codes) || misaligned(v_sz) || misaligned(k_res) || misaligned(v_res))
        return MINIKV_ERR_ALIGN;
    return status_of(minikv::launch_stream_step_append(k_new, v_new, B, Hkv, D, cap, counts, k_codes, k_sz, v_codes,
                                                       v_sz, k_res, v_res, as_stream(stream)));
}

size_t minikv_stream_step_decode_ws_bytes(int B, int Hq, int Hkv, int cap, int D) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || cap < MINIKV_GROUP || cap % MINIKV_GROUP || !supported_d(D))
        return 0;
    const minikv::DecodePlan plan = minikv::decode_plan(B, Hq, Hkv, cap, D);
    return minikv::stream_decode_ws_bytes(B, Hq, D, cap, MINIKV_GROUP - 1, plan);
}

int minikv_stream_step_decode(const void* q, int B, int Hq, int Hkv, int D, int cap, const int32_t* counts,
                              const uint8_t* k_codes, const uint32_t* k_sz, const uint8_t* v_codes,
                              const uint32_t* v_sz, const void* k_res, const void* v_res, float sm_scale, void* out,
                              void* ws, size_t ws_bytes, void* stream) {
    if (!q || !out || !counts || !k_codes || !k_sz || !v_codes || !v_sz || !k_res || !v_res || !ws)
        return MINIKV_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || cap < MINIKV_GROUP || cap % MINIKV_GROUP) return MINIKV_ERR_SHAPE;
    if (!supported_d(D)) return MINIKV_ERR_UNSUPPORTED;
    const int R = Hq / Hkv;
    if (R != 1 && R != 2 && R != 4) return MINIKV_ERR_UNSUPPORTED;
    if (misaligned(q) || misaligned(out) || misaligned(ws) || misaligned(counts) || misaligned(k_codes) ||
        misaligned(k_sz) || misaligned(v_codes) || misaligned(v_sz) || misaligned(k_res) || misaligned(v_res))
        return MINIKV_ERR_ALIGN;
    const minikv::DecodePlan plan = minikv::decode_plan(B, Hq, Hkv, cap, D);
    if (ws_bytes < minikv::stream_decode_ws_bytes(B, Hq, D, cap, MINIKV_GROUP - 1, plan)) return MINIKV_ERR_WORKSPACE;
    return status_of(minikv::launch_stream_decode_counted(q, k_codes, k_sz, v_codes, v_sz, B, Hq, Hkv, D, cap, counts,
                                                          k_res, v_res, resolve_scale(sm_scale, D), out, ws, plan,
                                                          as_stream(stream)));
}

}  // extern "C"
