// Whole-model attention driver: runs the hybrid layer schedule (layer l is full-causal iff
// l % 4 == 3, every other layer sliding-window) through the single-layer calls, and
// accounts the KV-cache bytes of that schedule.
// [T1] "Hybrid attention: only one layer in four gets the full view" (layers 3, 7, ..., 35
// are global); [T2] "27 sliding-window layers plus 9 global layers"; [T3] "36-layer hybrid
// layout"; [T1] "Doing the arithmetic first" (4096 bytes per token per layer).
//
// Host code only: every step is one of the library's kernels, launched on the caller's
// stream in layer order.  Nothing is allocated; the caller's workspace is reused by each
// layer in turn (stream order keeps the layers from overlapping).
#include <cstdint>

#include "../../include/hattn.h"
#include "hattn_device.h"
#include "hattn_launch.h"

namespace {

constexpr int32_t kMaxLayers = 4096;
constexpr int32_t kRing = 512;
constexpr size_t kRowBytes = (size_t)hattn::kHkv * hattn::kD * 2;  // one token's K (or V)

bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t kind_of(int32_t layer) { return layer % 4 == 3 ? HATTN_FULL : HATTN_SLIDING; }

// Pointers of every layer present and aligned (the per-layer calls repeat these checks;
// doing them first means a bad layer is reported before any layer is enqueued).
hattn_status check_layers(const hattn_layer_io* layers, int32_t n_layers) {
  for (int32_t l = 0; l < n_layers; ++l) {
    const hattn_layer_io& L = layers[l];
    if (!L.q || !L.k || !L.v || !L.gate || !L.k_cache || !L.v_cache || !L.out)
      return HATTN_ERR_NULL;
    if (!a16(L.q) || !a16(L.k) || !a16(L.v) || !a16(L.k_cache) || !a16(L.v_cache) ||
        !a16(L.out) || (reinterpret_cast<uintptr_t>(L.gate) & 1u) ||
        (L.lse && (reinterpret_cast<uintptr_t>(L.lse) & 3u)))
      return HATTN_ERR_ALIGN;
  }
  return HATTN_OK;
}

hattn_status check_common(const hattn_layer_io* layers, int32_t n_layers, int32_t B, int32_t cap) {
  // Batch is a grid dimension (y) of the per-layer launches, whose extent stops at 65535.
  if (n_layers < 1 || n_layers > kMaxLayers || B < 0 || B > 65535 || cap < kRing)
    return HATTN_ERR_SHAPE;
  if (layers == nullptr) return HATTN_ERR_NULL;
  return HATTN_OK;
}

// Decode workspace layout: the full layers' split partials, then (16-byte aligned) the
// sliding layers' ring-step partials and counters.
size_t full_region_bytes(int32_t n_layers, int32_t B, int32_t cap) {
  hattn_layer_cfg full;
  hattn_cfg_preset(HATTN_FULL, &full);
  const size_t need = n_layers > 3 ? hattn_decode_workspace_bytes(&full, B, cap) : 0;
  return (need + 15) & ~(size_t)15;
}

}  // namespace

extern "C" {

int32_t hattn_model_layer_kind(int32_t layer) { return layer < 0 ? -1 : kind_of(layer); }

hattn_status hattn_model_kv_bytes(int32_t n_layers, int32_t B, int32_t cap, size_t* per_layer,
                                  size_t* total) {
  if (n_layers < 1 || n_layers > kMaxLayers || B < 0 || cap < kRing) return HATTN_ERR_SHAPE;
  if (total == nullptr) return HATTN_ERR_NULL;
  size_t sum = 0;
  for (int32_t l = 0; l < n_layers; ++l) {
    const size_t rows = kind_of(l) == HATTN_FULL ? (size_t)cap : (size_t)kRing;
    const size_t bytes = 2 * (size_t)B * rows * kRowBytes;  // K and V
    if (per_layer) per_layer[l] = bytes;
    sum += bytes;
  }
  *total = sum;
  return HATTN_OK;
}

size_t hattn_model_decode_workspace_bytes(int32_t n_layers, int32_t B, int32_t cap) {
  if (n_layers < 1 || n_layers > kMaxLayers || B < 1 || B > 65535 || cap < kRing) return 0;
  return full_region_bytes(n_layers, B, cap) + hattn::ring_step_workspace_bytes(B);
}

hattn_status hattn_model_decode(const hattn_layer_io* layers, int32_t n_layers, int32_t cap,
                                const int32_t* pos, int32_t B, void* workspace,
                                size_t workspace_bytes, void* stream) {
  hattn_status st = check_common(layers, n_layers, B, cap);
  if (st != HATTN_OK) return st;
  if (B == 0) return HATTN_OK;
  if (pos == nullptr) return HATTN_ERR_NULL;
  st = check_layers(layers, n_layers);
  if (st != HATTN_OK) return st;
  const size_t need = hattn_model_decode_workspace_bytes(n_layers, B, cap);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return HATTN_ERR_WORKSPACE;
  if (!a16(workspace) || (reinterpret_cast<uintptr_t>(pos) & 3u)) return HATTN_ERR_ALIGN;
  hattn_layer_cfg sliding;
  hattn_cfg_preset(HATTN_SLIDING, &sliding);
  const hattn::RopeTable sliding_tab = hattn::rope_table(&sliding);
  const float sliding_scale = hattn::scale_log2e(&sliding);
  // Null when nothing needs a workspace (sliding layers only, at batches whose ring kernels
  // keep no partials).
  void* ring_ws = workspace == nullptr ? nullptr
                                       : static_cast<char*>(workspace) + full_region_bytes(n_layers, B, cap);
  {
    const hipError_t e = hattn::clear_ring_counters(ring_ws, B, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hattn::note_hip_error(e);
  }
  for (int32_t l = 0; l < n_layers; ++l) {
    const hattn_layer_io& L = layers[l];
    hattn_layer_cfg cfg;
    hattn_cfg_preset(kind_of(l), &cfg);
    if (cfg.kind == HATTN_SLIDING) {
      // Append, ring attention and merge in one launch.
      const hipError_t e = hattn::launch_ring_step(
          static_cast<const hattn::bf16_t*>(L.q), static_cast<const hattn::bf16_t*>(L.k),
          static_cast<const hattn::bf16_t*>(L.v), static_cast<hattn::bf16_t*>(L.k_cache),
          static_cast<hattn::bf16_t*>(L.v_cache), pos, B,
          static_cast<const hattn::bf16_t*>(L.gate), static_cast<hattn::bf16_t*>(L.out),
          static_cast<float*>(L.lse), sliding_tab, sliding_scale, ring_ws,
          reinterpret_cast<hipStream_t>(stream));
      if (e != hipSuccess) return hattn::note_hip_error(e);
      continue;
    }
    st = hattn_kv_append_rope(&cfg, L.k, L.v, L.k_cache, L.v_cache, cap, pos, B, 1, nullptr, stream);
    if (st != HATTN_OK) return st;
    st = hattn_decode(&cfg, L.q, L.k_cache, L.v_cache, cap, pos, B, L.gate, L.out, L.lse, workspace,
                      workspace_bytes, HATTN_ROPE_Q_FUSED, stream);
    if (st != HATTN_OK) return st;
  }
  return HATTN_OK;
}

size_t hattn_model_prefill_workspace_bytes(int32_t n_layers, int32_t B, int32_t Sq) {
  if (n_layers < 1 || n_layers > kMaxLayers || B < 1 || Sq < 1) return 0;
  return (size_t)B * (size_t)Sq * kRowBytes;  // one sliding layer's rotated chunk keys
}

hattn_status hattn_model_prefill(const hattn_layer_io* layers, int32_t n_layers, int32_t cap,
                                 const int32_t* pos0, int32_t B, int32_t Sq, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  hattn_status st = check_common(layers, n_layers, B, cap);
  if (st != HATTN_OK) return st;
  if (Sq < 0) return HATTN_ERR_SHAPE;
  if ((long long)B * Sq == 0) return HATTN_OK;
  if (pos0 == nullptr) return HATTN_ERR_NULL;
  st = check_layers(layers, n_layers);
  if (st != HATTN_OK) return st;
  const size_t need = hattn_model_prefill_workspace_bytes(n_layers, B, Sq);
  if (workspace == nullptr || workspace_bytes < need) return HATTN_ERR_WORKSPACE;
  if (!a16(workspace) || (reinterpret_cast<uintptr_t>(pos0) & 3u)) return HATTN_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (int32_t l = 0; l < n_layers; ++l) {
    const hattn_layer_io& L = layers[l];
    hattn_layer_cfg cfg;
    hattn_cfg_preset(kind_of(l), &cfg);
    if (cfg.kind == HATTN_FULL) {
      // The chunk's keys go into the position-indexed cache first; its queries then see
      // them there together with the whole history.
      st = hattn_kv_append_rope(&cfg, L.k, L.v, L.k_cache, L.v_cache, cap, pos0, B, Sq, nullptr,
                                stream);
      if (st != HATTN_OK) return st;
      st = hattn_prefill(&cfg, L.q, L.k_cache, L.v_cache, cap, pos0, B, Sq, L.gate, L.out, L.lse,
                         HATTN_ROPE_Q_FUSED, stream);
    } else {
      // Rotated chunk keys in the workspace; attend against the ring, then append (the ring
      // must not be overwritten before the chunk's earlier rows have read it).
      const hipError_t e = hipMemcpyAsync(workspace, L.k, need, hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return hattn::note_hip_error(e);
      st = hattn_rope_qk(&cfg, nullptr, workspace, pos0, B, Sq, stream);
      if (st != HATTN_OK) return st;
      st = hattn_prefill_ring(&cfg, L.q, workspace, L.v, L.k_cache, L.v_cache, pos0, B, Sq,
                              L.gate, L.out, L.lse, HATTN_ROPE_Q_FUSED, stream);
      if (st != HATTN_OK) return st;
      st = hattn_kv_append(&cfg, workspace, L.v, L.k_cache, L.v_cache, kRing, pos0, B, Sq, nullptr,
                           stream);
    }
    if (st != HATTN_OK) return st;
  }
  return HATTN_OK;
}

}  // extern "C"
