/*
 * minikv.h - C ABI of the MI355X (gfx950) library for attention over a 2-bit,
 * layer-discriminative KV cache.
 *
 * The method: "MiniKV: Pushing the Limits of LLM Inference via 2-Bit
 * Layer-Discriminative KV Cache" (paper-listing page, abstract: a 2-bit
 * layer-discriminative KV cache kept usable by FlashAttention-style kernels),
 * and the gptget.net summary of arXiv 2411.18077, sections 方法论 (methodology)
 * and 方法详解 (method details): 2-bit quantisation with an adaptive
 * (importance-based) KV policy, per-channel key quantisation, per-token value
 * quantisation, a compact cache layout, and "selective flash attention" built
 * from a second kernel.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are dense, row-major, with the shapes given per call.  Shape
 *    letters: B batch, T context tokens, Hq query heads, Hkv key/value heads
 *    (Hq % Hkv == 0; query head h reads KV head h / (Hq/Hkv)), D head dim
 *    (64 or 128), W observation-window rows, n_keep kept tokens.
 *  - Every data pointer is a DEVICE pointer owned by the caller; the library
 *    never allocates, frees or synchronises.  Pointers must be 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream); every
 *    call only enqueues work on it and returns.
 *  - Return value: MINIKV_OK (0) or a negative MINIKV_ERR_* status.  All
 *    argument checks run before any HIP call, so a rejected call has no effect
 *    and needs no GPU.  Faults inside kernels surface at the caller's next
 *    synchronisation of `stream`.
 *  - Stateless and reentrant; calls that write the same buffers must not
 *    overlap.
 *  - Preconditions not checked on the device: inputs are finite and
 *    |x| < 65504 (scales and zeros are stored in fp16).
 *  - One (sequence, head) slice of K or V, T rows of D elements, is at most
 *    2^31 - 1 bytes (the kernels address it through a 32-bit buffer range):
 *    T <= 8,388,607 for bf16 and 4,194,303 for fp32 at D = 128.  Calls that
 *    take such a slice return UNSUPPORTED beyond it.
 */
#ifndef MINIKV_H
#define MINIKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MINIKV_OK = 0,
    MINIKV_ERR_NULL = -1,        /* a required pointer is NULL */
    MINIKV_ERR_SHAPE = -2,       /* inconsistent or out-of-range sizes */
    MINIKV_ERR_UNSUPPORTED = -3, /* valid but not supported (D, group, dtype, T limit) */
    MINIKV_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
    MINIKV_ERR_WORKSPACE = -5,   /* workspace missing or too small */
    MINIKV_ERR_LAUNCH = -6       /* the HIP runtime rejected a kernel launch */
};

enum { MINIKV_F32 = 0, MINIKV_BF16 = 1 };

enum { MINIKV_GROUP = 32 };  /* quantisation group: 32 kept tokens (K) or 32 channels (V) */

/*
 * Packed 2-bit cache of n_keep tokens per (sequence, KV head): the "compact
 * layout" of the method-details section.  All four arrays are caller-owned
 * device buffers:
 *   k_codes  uint8 [B][Hkv][n_keep][D/4]         packed along channels: byte m of a token
 *                                                holds channels 4m..4m+3, channel 4m+j in bits 2j..2j+1
 *   k_sz     uint32[B][Hkv][G][D]                per channel, per block of 32 kept tokens
 *   v_codes  uint8 [B][Hkv][G][D][8]             packed along tokens: the 8 bytes of (block, channel)
 *                                                hold its 32 codes, token 4m+j of the block in bits
 *                                                2j..2j+1 of byte m; tokens past n_keep are code 0
 *   v_sz     uint32[B][Hkv][n_keep][D/32]        per token, per group of 32 channels
 * with G = ceil(n_keep/32).  A k_sz / v_sz word holds fp16 scale s in bits
 * 0..15 and fp16 zero z in bits 16..31; a code c stands for c*s + z.  Kept
 * tokens are stored in ascending position order; the last key group of a row
 * may hold fewer than 32 tokens.
 */
typedef struct {
    uint8_t *k_codes;
    uint32_t *k_sz;
    uint8_t *v_codes;
    uint32_t *v_sz;
    int32_t B, Hkv, n_keep, D, group; /* group must be MINIKV_GROUP */
} minikv_packed_t;

/*
 * Selective flash attention (method-details section: selective flash
 * attention from a second kernel; abstract: FlashAttention compatibility).
 *
 * Pass 1 - minikv_prefill_attn: causal attention over bf16 q [B][Hq][T][D],
 * k, v [B][Hkv][T][D]:
 *   o[b,h,i,:] = sum_{j<=i} softmax_j(q_i . k_j * sm_scale) v_j   (bf16 out, fp32 math)
 *   lse[b,h,i] = log sum_{j<=i} exp(q_i . k_j * sm_scale)            (fp32, natural log)
 * `o` may be NULL: only lse is written (the PV product is skipped).
 *
 * Pass 2 - minikv_window_scores (the second kernel): per-key probability mass
 * from the last W rows, summed over the query heads sharing a KV head:
 *   scores[b,g,j] = sum_{h: h/(Hq/Hkv)=g} sum_{i=T-W}^{T-1} [j<=i] exp(q_i . k_j * sm_scale - lse[b,h,i])
 * (fp32 [B][Hkv][T]); it needs lse only for rows T-W..T-1.  No T x T matrix is
 * stored by either pass.
 *
 * minikv_prefill_attn_scores computes both.  Where
 * minikv_prefill_fuses_scores(B, T, Hq, Hkv, W) is 1 (one query head per KV
 * head, W <= 32, the W rows inside the last 256-row query block, and at least
 * as many heads B * Hq as the device has compute units) it is a single
 * launch: the workgroup that finishes a head's last query block scores that
 * head's keys from its own lse right away, while K is still cached.  The
 * results are bit-identical to minikv_prefill_attn followed by
 * minikv_window_scores.  Otherwise it enqueues the two passes.
 * sm_scale <= 0 means 1/sqrt(D).
 * Errors: NULL q/k/v/lse/scores; SHAPE if any size < 1, Hq % Hkv, W > T;
 * UNSUPPORTED if D is not 64 or 128 or a K / V slice exceeds 2 GiB; ALIGN;
 * LAUNCH.
 * minikv_prefill_fuses_scores returns 1 or 0 (0 for invalid sizes too); its
 * only HIP call is a query of the current device's compute-unit count (256
 * is assumed when there is no device).
 */
int minikv_prefill_attn(const void *q, const void *k, const void *v,
                        int B, int T, int Hq, int Hkv, int D, float sm_scale,
                        void *o, float *lse, void *stream);

int minikv_window_scores(const void *q, const void *k, const float *lse,
                         int B, int T, int Hq, int Hkv, int D, int window,
                         float sm_scale, float *scores, void *stream);

int minikv_prefill_attn_scores(const void *q, const void *k, const void *v,
                               int B, int T, int Hq, int Hkv, int D, int window,
                               float sm_scale, void *o, float *lse, float *scores,
                               void *stream);

int minikv_prefill_fuses_scores(int B, int T, int Hq, int Hkv, int window);

/*
 * Heavy-hitter + recent-window selection (gptget.net summary, 术语表 "adaptive
 * KV": keep the KV states chosen by importance).
 * scores fp32 [B][Hkv][T] (non-negative) -> idx int32 [B][Hkv][n_heavy+n_recent]:
 * positions T-n_recent..T-1 plus the n_heavy largest scores among positions
 * < T-n_recent (equal scores: the lower position first), ascending.
 * ws: device workspace of at least minikv_select_ws_bytes(B, Hkv, T) bytes,
 * caller-owned; when that size is 0 (every supported shape today: one
 * workgroup per row keeps its keys and histograms on chip) ws may be NULL and
 * ws_bytes 0.
 * Errors: NULL (scores, idx); SHAPE if n_heavy<0, n_recent<0,
 * n_heavy+n_recent<1 or > T; UNSUPPORTED if T - n_recent > 65536; ALIGN;
 * WORKSPACE; LAUNCH.
 */
int minikv_select_topk(const float *scores, int B, int Hkv, int T,
                       int n_heavy, int n_recent, int32_t *idx,
                       void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes minikv_select_topk needs (0 also for invalid sizes). */
size_t minikv_select_ws_bytes(int B, int Hkv, int T);

/*
 * 2-bit asymmetric min/max quantise-and-pack of the kept tokens (method
 * details: per-channel key and per-token value quantisation, compact layout).
 * k, v [B][Hkv][T][D] in fp32 (in_dtype MINIKV_F32) or bf16 (MINIKV_BF16);
 * idx int32 [B][Hkv][n_keep] ascending positions (NULL keeps every token,
 * n_keep must then equal T).  Per group (32 kept tokens x 1 channel for K,
 * 1 token x 32 channels for V), in IEEE fp32 with round-half-even:
 *   s = fp16(fl32(max - min) / 3), z = fp16(min),
 *   code = s == 0 ? 0 : clamp(rint(fl32(x - z) / s), 0, 3)
 * with the stored fp16 s, z; a short last K group uses its valid tokens only.
 * Errors: NULL; SHAPE (sizes < 1, n_keep > T, out->B/Hkv/n_keep/D mismatch,
 * idx NULL with n_keep != T); UNSUPPORTED (D, group != 32, in_dtype, a K / V
 * slice over 2 GiB); ALIGN; LAUNCH.  idx entries outside [0, T) are not
 * checked on the device (such rows read as zeros).
 */
int minikv_quant_pack(const void *k, const void *v, int in_dtype, const int32_t *idx,
                      int B, int Hkv, int T, int D, int n_keep,
                      const minikv_packed_t *out, void *stream);

/*
 * Single-query decode attention over the packed cache, dequantising in
 * registers (abstract: the compressed cache serves inference).
 * q bf16 [B][Hq][D] -> out bf16 [B][Hq][D]:
 *   out[b,h] = sum_t softmax_t(q . khat_t * sm_scale) vhat_t over the n_keep packed tokens,
 * khat / vhat = code * s + z.  ws: device workspace of at least
 * minikv_decode_ws_bytes(B, Hq, Hkv, n_keep, D) bytes.  Its first
 * MINIKV_DECODE_TICKET_BYTES bytes must hold zeros before the buffer's first
 * use by any decode call: a head whose tokens are split over several
 * workgroups takes a ticket there, the last workgroup merges the head's
 * parts (which follow the tickets), and every call leaves the tickets zero
 * again.  sm_scale <= 0 means 1/sqrt(D).
 * Errors: NULL; SHAPE (Hq % cache->Hkv, sizes < 1); UNSUPPORTED (D, group,
 * Hq/Hkv not 1, 2 or 4); ALIGN; WORKSPACE; LAUNCH.
 */
#define MINIKV_DECODE_TICKET_BYTES ((size_t)16384)
int minikv_decode_attn(const void *q, const minikv_packed_t *cache, int Hq, float sm_scale,
                       void *out, void *ws, size_t ws_bytes, void *stream);

/*
 * For callers that cannot allocate device memory - code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc:
 * minikv_decode_attn without a workspace argument.  The split partial results
 * go to a library-owned device array of MINIKV_DECODE_SCRATCH_BYTES on each
 * GPU the library runs on, held until the process ends; no hipMalloc,
 * hipFree or allocating routine is called.  Same arguments (minus ws),
 * results and errors as minikv_decode_attn, plus WORKSPACE when the split
 * plan's workspace (minikv_decode_ws_bytes) exceeds the array - no plan of a
 * supported shape does: at most about 8192 (KV head, part) pairs of (D + 2)
 * floats per query head, 17 MB at four query heads per KV head and D = 128,
 * after the tickets; a plan with one range per KV head uses no scratch - and
 * LAUNCH when the array's device address cannot be resolved.
 * Every call on a GPU shares that GPU's array: its tickets start at zero
 * (the array is zero-initialised) and every call leaves them zero; the parts
 * keep the last call's values.  Calls that overlap on one GPU (other
 * streams, other threads) race.
 */
#define MINIKV_DECODE_SCRATCH_BYTES ((size_t)32 << 20)
int minikv_decode_attn_noalloc(const void *q, const minikv_packed_t *cache, int Hq, float sm_scale,
                               void *out, void *stream);

/* ---- streaming decode: generated tokens join the cache ----
 *
 * Keys are quantised per channel over 32-token groups (method details), so a
 * key group needs 32 whole tokens.  Streaming layout per (sequence, KV head):
 *   - a packed region laid out for `cap` tokens (cap a multiple of 32):
 *       k_codes [B][Hkv][cap][D/4], k_sz [B][Hkv][cap/32][D],
 *       v_codes [B][Hkv][cap/32][D][8], v_sz [B][Hkv][cap][D/32]
 *     (the minikv_quant_pack layout with cap in place of n_keep), of which the
 *     first n_packed tokens (a multiple of 32) are valid;
 *   - a residual window k_res, v_res bf16 [B][Hkv][32][D] whose first n_res
 *     (0..31) slots hold tokens kept exactly.
 * A selection of n_keep tokens starts with its first 32*floor(n_keep/32)
 * tokens packed (minikv_stream_pack) and the rest in the window
 * (minikv_stream_append with idx).  Each generated token is appended to the
 * window; when the window holds 32 tokens the caller packs it at token
 * n_packed (minikv_stream_pack, idx NULL, T = 32) and empties it.  The caller
 * owns every buffer and tracks n_packed and n_res (all sequences of a batch
 * advance together).
 */

/*
 * Quantise-and-pack n tokens (n and tok0 multiples of 32, tok0 + n <= cap)
 * into tokens tok0 .. tok0+n-1 of a streaming layout for cap tokens.  Source:
 * k, v [B][Hkv][T][D] (in_dtype as for minikv_quant_pack), rows idx[b][g][j]
 * (int32, row stride idx_stride >= n) or, with idx NULL, rows 0..n-1 (n <= T).
 * Same rule as minikv_quant_pack; the packed bytes of whole groups do not
 * depend on where they are placed.
 * Errors: NULL; SHAPE (sizes < 1, n or tok0 not multiples of 32, tok0 + n > cap,
 * cap not a multiple of 32, idx_stride < n, n > T with idx NULL);
 * UNSUPPORTED (D, in_dtype, a K / V slice over 2 GiB); ALIGN; LAUNCH.
 */
int minikv_stream_pack(const void *k, const void *v, int in_dtype, const int32_t *idx, int idx_stride,
                       int B, int Hkv, int T, int D, int n, int cap, int tok0,
                       uint8_t *k_codes, uint32_t *k_sz, uint8_t *v_codes, uint32_t *v_sz,
                       void *stream);

/*
 * Copy n bf16 tokens into residual slots slot .. slot+n-1 (slot + n <= 32) of
 * k_res, v_res bf16 [B][Hkv][32][D]: rows idx[b][g][j] (row stride idx_stride)
 * of k, v bf16 [B][Hkv][T][D], or rows 0..n-1 with idx NULL (a generated token:
 * T = 1, n = 1).  Errors: NULL; SHAPE; UNSUPPORTED (D, a K / V slice over
 * 2 GiB); ALIGN; LAUNCH.
 */
int minikv_stream_append(const void *k, const void *v, const int32_t *idx, int idx_stride,
                         int B, int Hkv, int T, int D, int n, int slot,
                         void *k_res, void *v_res, void *stream);

/*
 * Single-query decode over a streaming cache: the softmax runs over the
 * n_packed packed tokens (dequantised in registers, as minikv_decode_attn)
 * and the n_res residual tokens (exact) together.  q bf16 [B][Hq][D] -> out
 * bf16 [B][Hq][D].  ws: at least minikv_stream_decode_ws_bytes(...) bytes,
 * whose first MINIKV_DECODE_TICKET_BYTES bytes hold zeros before the buffer's
 * first use, as for minikv_decode_attn (when a KV head's tokens are split over
 * a few workgroups the window's exact part is merged in the same launch as
 * the packed tokens, by the head's last workgroup).
 * sm_scale <= 0 means 1/sqrt(D).
 * Errors: NULL; SHAPE (Hq % Hkv, n_packed not a multiple of 32 or > cap,
 * n_res outside 0..31, n_packed + n_res < 1); UNSUPPORTED (D, Hq/Hkv not 1,
 * 2 or 4); ALIGN; WORKSPACE; LAUNCH.
 */
int minikv_stream_decode(const void *q, int B, int Hq, int Hkv, int D, int cap, int n_packed,
                         const uint8_t *k_codes, const uint32_t *k_sz, const uint8_t *v_codes,
                         const uint32_t *v_sz, const void *k_res, const void *v_res, int n_res,
                         float sm_scale, void *out, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes minikv_stream_decode needs (0 for invalid sizes). */
size_t minikv_stream_decode_ws_bytes(int B, int Hq, int Hkv, int n_packed, int n_res, int D);

/*
 * The same two operations with the decisions taken here and the host-side
 * counts kept in caller-owned ints (bf16 K/V; streaming layout as above).
 *
 * minikv_stream_init starts a cache from a selection idx int32 [B][Hkv][n_keep]
 * (ascending, row stride n_keep) of k, v bf16 [B][Hkv][T][D]: the first
 * 32*floor(n_keep/32) selected tokens are packed at token 0, the remaining
 * n_keep mod 32 are copied into window slots 0.., and *n_packed, *n_res are
 * set to those two counts.  Errors: NULL (any pointer); SHAPE (sizes < 1,
 * n_keep > T, cap not a positive multiple of 32, the packed part > cap);
 * UNSUPPORTED (D, a K / V slice over 2 GiB); ALIGN; LAUNCH.  On an error nothing is enqueued (LAUNCH
 * aside) and the counts are unchanged.
 *
 * minikv_stream_append_token appends k_new, v_new bf16 [B][Hkv][D] into window
 * slot *n_res; when that token fills the window the window is packed at token
 * *n_packed (the minikv_stream_pack rule) and emptied.  The counts advance
 * (*n_res + 1, or *n_packed + 32 and *n_res = 0).  Errors: NULL; SHAPE (sizes,
 * counts out of range, or the window would have to be packed past cap: then
 * nothing is enqueued and the counts are unchanged); UNSUPPORTED (D); ALIGN;
 * LAUNCH.
 */
int minikv_stream_init(const void *k, const void *v, const int32_t *idx, int B, int Hkv, int T, int D,
                       int n_keep, int cap, uint8_t *k_codes, uint32_t *k_sz, uint8_t *v_codes,
                       uint32_t *v_sz, void *k_res, void *v_res, int *n_packed, int *n_res, void *stream);

int minikv_stream_append_token(const void *k_new, const void *v_new, int B, int Hkv, int D, int cap,
                               int *n_packed, int *n_res, uint8_t *k_codes, uint32_t *k_sz,
                               uint8_t *v_codes, uint32_t *v_sz, void *k_res, void *v_res, void *stream);

/*
 * A generation step with the counts in device memory, so that the step is a
 * fixed sequence of launches a HIP graph can capture and replay (the host no
 * longer passes n_packed / n_res).  counts: device int32[4], caller-owned,
 * {n_packed, n_res, overflow flag, ticket}; the same streaming layout as above.
 *
 * minikv_stream_set_counts writes {n_packed, n_res, 0, 0} with a kernel (no
 * memset node).  Errors: NULL; SHAPE (cap not a positive multiple of 32,
 * n_packed not a multiple of 32 or > cap, n_res outside 0..31); ALIGN; LAUNCH.
 *
 * minikv_stream_step_append appends k_new, v_new bf16 [B][Hkv][D] (one token
 * per sequence and KV head) in one launch: the token into window slot n_res;
 * the window packed at token n_packed when that token filled it (the same
 * quantisation as minikv_stream_pack); counts advanced (n_res + 1, or
 * n_packed + 32 and n_res = 0 after a pack) by the workgroup that finishes
 * last (counts[3] is its ticket and is back at 0 after every call).  When a full window cannot be
 * packed (n_packed + 32 > cap) the overflow flag is set, the window is kept,
 * and every later step writes nothing until the counts are set again: the
 * caller reads the flag to detect it.  Errors: NULL; SHAPE (sizes, cap);
 * UNSUPPORTED (D); ALIGN; LAUNCH.
 *
 * minikv_stream_step_decode is minikv_stream_decode with the counts read on
 * the device: the split plan covers all cap tokens (token ranges past n_packed
 * contribute empty parts) and the window is always a part (empty at n_res 0).
 * Workspace: minikv_stream_step_decode_ws_bytes (0 for invalid sizes), its
 * first MINIKV_DECODE_TICKET_BYTES bytes zero before first use (every call
 * leaves them zero).
 * Errors: NULL (any pointer, ws included); SHAPE; UNSUPPORTED (D, Hq/Hkv not
 * 1, 2 or 4); ALIGN; WORKSPACE; LAUNCH.  Calls that overlap on one counts
 * buffer race.
 */
int minikv_stream_set_counts(int32_t *counts, int n_packed, int n_res, int cap, void *stream);

int minikv_stream_step_append(const void *k_new, const void *v_new, int B, int Hkv, int D, int cap,
                              int32_t *counts, uint8_t *k_codes, uint32_t *k_sz, uint8_t *v_codes,
                              uint32_t *v_sz, void *k_res, void *v_res, void *stream);

size_t minikv_stream_step_decode_ws_bytes(int B, int Hq, int Hkv, int cap, int D);

int minikv_stream_step_decode(const void *q, int B, int Hq, int Hkv, int D, int cap, const int32_t *counts,
                              const uint8_t *k_codes, const uint32_t *k_sz, const uint8_t *v_codes,
                              const uint32_t *v_sz, const void *k_res, const void *v_res, float sm_scale,
                              void *out, void *ws, size_t ws_bytes, void *stream);

/* ---- host helpers (no GPU work) ---- */

/* Bytes of the packed cache: per (sequence, KV head), G = ceil(n/32):
 * n*D/4 + G*D*4 + G*32*D/4 + n*(D/32)*4.  Returns 0 for invalid sizes. */
size_t minikv_packed_bytes(int B, int Hkv, int n_keep, int D);

/* Workspace bytes minikv_decode_attn needs for this shape (0 for invalid sizes). */
size_t minikv_decode_ws_bytes(int B, int Hq, int Hkv, int n_keep, int D);

/* Kept tokens at a budget of pct_milli/1000 percent of T: floor(pct*T/100), at least 1.
 * (Glossary "adaptive KV".)  Returns a negative status for T < 1 or pct outside (0, 100]. */
int minikv_keep_count(int T, int pct_milli);

/* Kept tokens of `layer` of an n_layers-deep layer-discriminative ("Pyramid",
 * notesum.ai LongBench table) cache whose budget falls linearly from first_pct %
 * at layer 0 to last_pct % at the last layer:
 * floor((first*(L-1) + (last-first)*layer) * T / (100*(L-1))), at least 1. */
int minikv_pyramid_keep(int T, int n_layers, int layer, int first_pct, int last_pct);

/* Split a budget into heavy and recent parts: recent = floor(n_keep/5). */
int minikv_split_heavy_recent(int n_keep, int *n_heavy, int *n_recent);

/* Static description of a status code. */
const char *minikv_status_string(int status);

/*
 * Measurement aid, not a step of the method: a streaming read of `bytes` bytes
 * at src (device, 16-byte aligned, a multiple of 16 bytes), whose rate is the
 * measured reference for the HBM-bound kernels' rooflines.  Every 16-byte
 * piece is read once (non-temporal loads); the XOR of the 32-bit words each
 * wave read goes to sink (device uint32 [MINIKV_READ_PROBE_SINK_WORDS],
 * caller-owned, 16-byte aligned; words past the launch's waves are left
 * untouched, so a zeroed sink XORs to the XOR of every word of the buffer).  Errors: NULL; SHAPE (bytes 0 or not a multiple
 * of 16); ALIGN; LAUNCH.
 */
#define MINIKV_READ_PROBE_SINK_WORDS 131072
int minikv_read_probe(const void *src, size_t bytes, uint32_t *sink, void *stream);

/* Identity of the library binary: "sha256:" and the first 16 hex digits of a hash of
 * every kernel and header source it was compiled from (static string). */
const char *minikv_build_id(void);

#ifdef __cplusplus
}
#endif

#endif /* MINIKV_H */
