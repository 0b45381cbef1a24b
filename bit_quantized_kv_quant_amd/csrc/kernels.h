// Internal launchers, one per kernel file.  Arguments are validated by the
// C-ABI layer (api.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace minikv {

// Compute units of the current device (cached on first use; 256 without a device).
int device_cu_count();

hipError_t launch_quant_pack(const void* k, const void* v, bool bf16, const int32_t* idx, int B,
                             int Hkv, int T_ctx, int D, int n_keep, uint8_t* k_codes, uint32_t* k_sz,
                             uint8_t* v_codes, uint32_t* v_sz, hipStream_t stream);

// Streaming: pack n tokens (selection idx with row stride idx_stride, or the
// first n rows) into tokens tok0.. of a layout for cap tokens per head.
hipError_t launch_stream_pack(const void* k, const void* v, bool bf16, const int32_t* idx, int idx_stride, int B,
                              int Hkv, int T_ctx, int D, int n, int cap, int tok0, uint8_t* k_codes,
                              uint32_t* k_sz, uint8_t* v_codes, uint32_t* v_sz, hipStream_t stream);

// Streaming: copy n bf16 rows (idx or the first n) into residual slots slot.. (32 per head).
hipError_t launch_stream_append(const void* k, const void* v, const int32_t* idx, int idx_stride, int B, int Hkv,
                                int T_ctx, int D, int n, int slot, void* k_res, void* v_res, hipStream_t stream);

// Device-side generation step (counts = device int32 {n_packed, n_res,
// overflow, ticket}): set the counts; in one launch, append one token per
// (sequence, KV head) into window slot n_res, pack a filled window at n_packed
// and advance the counts.
hipError_t launch_stream_set_counts(int32_t* counts, int n_packed, int n_res, hipStream_t stream);
hipError_t launch_stream_step_append(const void* k_new, const void* v_new, int B, int Hkv, int D, int cap,
                                     int32_t* counts, uint8_t* k_codes, uint32_t* k_sz, uint8_t* v_codes,
                                     uint32_t* v_sz, void* k_res, void* v_res, hipStream_t stream);

hipError_t launch_select_topk(const float* scores, int B, int Hkv, int T_ctx, int n_heavy,
                              int n_recent, int32_t* idx, hipStream_t stream);

// Decode: split plan shared by the workspace-size query and the launcher.
struct DecodePlan {
    int splits;   // token ranges per (sequence, KV head)
    int chunk;    // tokens per split (multiple of 128)
    bool ticket;  // a split head merged inside the launch (splits a multiple of nw)
    int nw;       // waves (token ranges) per workgroup of such a launch: 4 or 8
};
// Most workgroups of ranges per head merged inside the decode launch
// (workgroup parts handed over by a ticket); heads split further use the
// separate merge kernel.  Measured: 7 workgroups of 8 ranges per head (a
// 6600-token head, 4 x 8 KV heads) merge faster in the launch than through
// the merge kernel (0.47 against 0.52 ms per 32-layer step); 13 workgroups
// of 4 ranges were slower (0.56).
constexpr int kTicketMaxWorkgroups = 8;
DecodePlan decode_plan(int B, int Hq, int Hkv, int n_keep, int D);
size_t decode_ws_bytes(int B, int Hq, int D, const DecodePlan& plan);
size_t stream_decode_ws_bytes(int B, int Hq, int D, int n_packed, int n_res, const DecodePlan& plan);

// Head of every decode workspace: one int32 ticket per (sequence, KV head)
// of a split plan (split plans have fewer than 4096 such heads).  It must
// hold zeros before a workspace's first use; every decode leaves it zero.
constexpr size_t kTicketBytes = 4096 * sizeof(int32_t);
// Bytes of the allocation-free decode's scratch array (one per device).
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
// Device address of the current device's scratch array (resolved once per
// device), or nullptr if the runtime cannot resolve it.
void* decode_scratch();

hipError_t launch_decode(const void* q, const uint8_t* k_codes, const uint32_t* k_sz,
                         const uint8_t* v_codes, const uint32_t* v_sz, int B, int Hq, int Hkv,
                         int n_keep, int D, float sm_scale, void* out, void* ws,
                         const DecodePlan& plan, hipStream_t stream);

// Streaming decode: n_packed tokens of a layout for cap tokens per head, then
// n_res exact residual tokens (bf16, 32 slots per head).
hipError_t launch_stream_decode(const void* q, const uint8_t* k_codes, const uint32_t* k_sz, const uint8_t* v_codes,
                                const uint32_t* v_sz, int B, int Hq, int Hkv, int D, int cap, int n_packed,
                                const void* k_res, const void* v_res, int n_res, float sm_scale, void* out,
                                void* ws, const DecodePlan& plan, hipStream_t stream);

// Pass 1; with window > 0 (only where prefill_fuses_scores) it also writes the
// window scores of pass 2 in the same launch.
bool prefill_fuses_scores(int B, int T_ctx, int Hq, int Hkv, int window);
// Streaming decode with the counts read on the device: planned for the whole
// capacity (plan of cap tokens), always a residual part.
hipError_t launch_stream_decode_counted(const void* q, const uint8_t* k_codes, const uint32_t* k_sz,
                                        const uint8_t* v_codes, const uint32_t* v_sz, int B, int Hq, int Hkv, int D,
                                        int cap, const int32_t* counts, const void* k_res, const void* v_res,
                                        float sm_scale, void* out, void* ws, const DecodePlan& plan,
                                        hipStream_t stream);

hipError_t launch_prefill(const void* q, const void* k, const void* v, int B, int T_ctx, int Hq,
                          int Hkv, int D, float sm_scale, void* o, float* lse, int window, float* scores,
                          hipStream_t stream);

hipError_t launch_window_scores(const void* q, const void* k, const float* lse, int B, int T_ctx,
                                int Hq, int Hkv, int D, int window, float sm_scale, float* scores,
                                hipStream_t stream);

// Streaming-read reference (measurement aid): sink_words / 4 workgroups of 256 threads.
hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int sink_words, hipStream_t stream);

}  // namespace minikv
