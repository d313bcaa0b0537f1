// Host-side launchers of the hattn kernels (called by the C ABI in api.hip after it has
// validated every argument).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "hattn_device.h"

struct hattn_layer_cfg;  // the C ABI's layer configuration

namespace hattn {

// Record e as the calling thread's last HIP error and return HATTN_ERR_HIP (api.hip).
int32_t note_hip_error(hipError_t e);

hipError_t launch_rope_qk(bf16_t* q, bf16_t* k, const int* pos0, int B, int S,
                          const RopeTable& tab, hipStream_t stream);

// rope_k: NULL copies k_new as given; otherwise each key is rotated by its position with
// this table while it is copied (k_new itself is not modified).
hipError_t launch_kv_append(const bf16_t* k_new, const bf16_t* v_new, bf16_t* k_cache,
                            bf16_t* v_cache, int cap, const int* pos0, int B, int n,
                            int window, int* slots_out, const RopeTable* rope_k,
                            hipStream_t stream);

// 8-bit KV append: caches [B, cap, 4, 256] E4M3 codes, scales [B, 4, cap] fp32.
hipError_t launch_kv_append_fp8(const bf16_t* k_new, const bf16_t* v_new, uint8_t* k_cache,
                                uint8_t* v_cache, float* k_scale, float* v_scale, int cap,
                                const int* pos0, int B, int n, int window, int* slots_out,
                                const RopeTable* rope_k, hipStream_t stream);

// window == 0 selects the full-causal kernel.
hipError_t launch_prefill(const bf16_t* q, const bf16_t* k_cache, const bf16_t* v_cache,
                          int cap, const int* pos0, int B, int Sq, const bf16_t* gate,
                          bf16_t* out, float* lse, int window, bool rope_q,
                          const RopeTable& tab, float scale_log2e, hipStream_t stream);

// Sliding-layer chunk that continues a 512-slot ring: k_new / v_new [B, Sq, 4, 256] hold
// the chunk's keys, k_ring / v_ring [B, 512, 4, 256] the older positions.
hipError_t launch_prefill_ring(const bf16_t* q, const bf16_t* k_new, const bf16_t* v_new,
                               const bf16_t* k_ring, const bf16_t* v_ring, const int* pos0, int B,
                               int Sq, const bf16_t* gate, bf16_t* out, float* lse, int window,
                               bool rope_q, const RopeTable& tab, float scale_log2e,
                               hipStream_t stream);

// RoPE inverse frequencies and the softmax scale times log2(e) of a validated layer
// configuration (the ABI layer builds these for every call).
RopeTable rope_table(const ::hattn_layer_cfg* cfg);
float scale_log2e(const ::hattn_layer_cfg* cfg);

// Split-KV decode geometry, a pure function of (B, max keys per sequence).
struct DecodePlan {
  int nchunks;  // key chunks per sequence
  int chunk;    // keys per chunk (multiple of 32)
};
DecodePlan decode_plan(int B, int max_keys);
size_t decode_workspace_bytes(int B, const DecodePlan& plan);

hipError_t launch_decode(const bf16_t* q, const bf16_t* k_cache, const bf16_t* v_cache, int cap,
                         const int* pos, int B, const bf16_t* gate, bf16_t* out, float* lse,
                         int window, bool rope_q, const RopeTable& tab, float scale_log2e,
                         const DecodePlan& plan, void* workspace, hipStream_t stream);

// One decode step of a sliding layer in one launch: rotate K by pos and append K / V at
// ring slot pos mod 512 of k_ring / v_ring [B, 512, 4, 256], then attend (Q-RoPE fused),
// gate and store out [B, 1, 16, 256] (and lse [B, 1, 16] unless null).  q, k_new, v_new
// are the token's un-rotated projections [B, 1, *, 256].  The ring is split over 8
// workgroups per (sequence, KV head) for B <= 8, 4 above, and workspace (16-byte aligned,
// at least ring_step_workspace_bytes(B) bytes) holds their partials and one counter per
// (sequence, KV head), which must be zero before the first step (clear_ring_counters) and
// which every step leaves at zero.
size_t ring_step_workspace_bytes(int B);
// The ring attention of a plain sliding decode (the token's key and value already in the
// ring; q rotated unless rope_q), for every B >= 1: it clears the split kernel's counters
// and launches it, in that order, on `stream`.
hipError_t launch_ring_decode(const bf16_t* q, const bf16_t* k_ring, const bf16_t* v_ring,
                              const int* pos, int B, const bf16_t* gate, bf16_t* out, float* lse,
                              bool rope_q, const RopeTable& tab, float scale_log2e,
                              void* workspace, hipStream_t stream);
hipError_t clear_ring_counters(void* workspace, int B, hipStream_t stream);
hipError_t launch_ring_step(const bf16_t* q, const bf16_t* k_new, const bf16_t* v_new,
                            bf16_t* k_ring, bf16_t* v_ring, const int* pos, int B,
                            const bf16_t* gate, bf16_t* out, float* lse, const RopeTable& tab,
                            float scale_log2e, void* workspace, hipStream_t stream);

// 8-bit KV decode: caches [B, cap, 4, 256] E4M3 codes, scales [B, 4, cap] fp32; same plan
// and workspace as launch_decode.
hipError_t launch_decode_fp8(const bf16_t* q, const uint8_t* k_cache, const uint8_t* v_cache,
                             const float* k_scale, const float* v_scale, int cap, const int* pos,
                             int B, const bf16_t* gate, bf16_t* out, float* lse, int window,
                             bool rope_q, const RopeTable& tab, float scale_log2e,
                             const DecodePlan& plan, void* workspace, hipStream_t stream);

// Fused QKV + gate projection: x [T, 2560] @ [w_qkv; w_gate]^T written as q [T,16,256],
// k / v [T,4,256] and gate logits [T,16]; w_qkv [6144, 2560], w_gate [16, 2560].
hipError_t launch_qkv_proj(const bf16_t* x, int T, const bf16_t* w_qkv, const bf16_t* w_gate,
                           bf16_t* q, bf16_t* k, bf16_t* v, bf16_t* gate, hipStream_t stream);
// Output projection: a [T, 4096] @ w_o^T, w_o [2560, 4096] -> y [T, 2560].
hipError_t launch_o_proj(const bf16_t* a, int T, const bf16_t* w_o, bf16_t* y,
                         hipStream_t stream);

}  // namespace hattn
