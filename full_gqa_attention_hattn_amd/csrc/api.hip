// C ABI of libhattn: argument validation, RoPE frequency tables and kernel dispatch.
// Every check runs on the host before anything is enqueued; kernels add their own range
// guards for the device-resident position arrays.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/hattn.h"
#include "hattn_device.h"
#include "hattn_launch.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

constexpr int32_t kWindow = 512;
constexpr float kLog2e = 1.44269504088896340736f;
// Largest number of work-items a one-dimensional launch may address.
constexpr long long kMaxWorkItems = 0xffffffffLL;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool aligned2(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 1u) == 0; }

hattn_layer_cfg preset(int32_t kind) {
  hattn_layer_cfg c{};
  c.kind = kind;
  c.n_q_heads = hattn::kHq;
  c.n_kv_heads = hattn::kHkv;
  c.head_dim = hattn::kD;
  c.softmax_scale = 1.0f / 16.0f;
  c.reserved = 0;
  if (kind == HATTN_SLIDING) {
    // [T3] "Sliding window 512": window 512, theta 1e4, all 256 dims rotate.
    c.window = kWindow;
    c.rot_dim = 256;
    c.rope_theta = 1.0e4;
  } else {
    // [T3] "Global attention + 5M-base RoPE": theta 5e6, first 64 of 256 dims rotate.
    c.window = 0;
    c.rot_dim = 64;
    c.rope_theta = 5.0e6;
  }
  return c;
}

hattn_status check_cfg(const hattn_layer_cfg* cfg) {
  if (cfg == nullptr) return HATTN_ERR_NULL;
  if (cfg->kind != HATTN_SLIDING && cfg->kind != HATTN_FULL) return HATTN_ERR_UNSUPPORTED;
  const hattn_layer_cfg p = preset(cfg->kind);
  if (cfg->n_q_heads != p.n_q_heads || cfg->n_kv_heads != p.n_kv_heads ||
      cfg->head_dim != p.head_dim || cfg->window != p.window || cfg->rot_dim != p.rot_dim ||
      cfg->rope_theta != p.rope_theta || cfg->softmax_scale != p.softmax_scale ||
      cfg->reserved != 0)
    return HATTN_ERR_UNSUPPORTED;
  return HATTN_OK;
}


hattn_status hip_status(hipError_t e) {
  if (e == hipSuccess) return HATTN_OK;
  g_last_hip_error = (int32_t)e;
  return HATTN_ERR_HIP;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int decode_max_keys(const hattn_layer_cfg* cfg, int32_t cap) {
  return cfg->kind == HATTN_SLIDING ? cfg->window : cap;
}

// Workspace a decode needs: full layers, the split-KV partials; sliding layers, the ring
// split's partials and counters.
size_t decode_need(const hattn_layer_cfg* cfg, int32_t B, int32_t cap) {
  if (cfg->kind == HATTN_SLIDING) return hattn::ring_step_workspace_bytes(B);
  return hattn::decode_workspace_bytes(B, hattn::decode_plan(B, decode_max_keys(cfg, cap)));
}

}  // namespace

namespace hattn {
RopeTable rope_table(const ::hattn_layer_cfg* cfg) {
  RopeTable t{};
  t.rot_dim = cfg->rot_dim;
  for (int i = 0; i < cfg->rot_dim / 2; ++i)
    t.inv_freq[i] = (float)std::pow(cfg->rope_theta, -2.0 * i / (double)cfg->rot_dim);
  return t;
}

float scale_log2e(const ::hattn_layer_cfg* cfg) { return cfg->softmax_scale * kLog2e; }
}  // namespace hattn

using hattn::rope_table;
using hattn::scale_log2e;

int32_t hattn::note_hip_error(hipError_t e) { return hip_status(e == hipSuccess ? hipErrorUnknown : e); }

extern "C" {

hattn_status hattn_cfg_preset(int32_t kind, hattn_layer_cfg* out) {
  if (out == nullptr) return HATTN_ERR_NULL;
  if (kind != HATTN_SLIDING && kind != HATTN_FULL) return HATTN_ERR_UNSUPPORTED;
  *out = preset(kind);
  return HATTN_OK;
}

hattn_status hattn_rope_qk(const hattn_layer_cfg* cfg, void* q, void* k, const int32_t* pos0,
                           int32_t B, int32_t S, void* stream) {
  hattn_status st = check_cfg(cfg);
  if (st != HATTN_OK) return st;
  if (B < 0 || S < 0) return HATTN_ERR_SHAPE;
  const long long ntok = (long long)B * S;
  if (ntok == 0) return HATTN_OK;
  if ((q == nullptr && k == nullptr) || pos0 == nullptr) return HATTN_ERR_NULL;
  if ((q && !aligned16(q)) || (k && !aligned16(k)) || !aligned4(pos0)) return HATTN_ERR_ALIGN;
  if (ntok * hattn::kHq * hattn::kD >= (1LL << 62) || (ntok + 3) / 4 * 256 > kMaxWorkItems)
    return HATTN_ERR_SHAPE;
  const hattn::RopeTable tab = rope_table(cfg);
  return hip_status(hattn::launch_rope_qk(static_cast<hattn::bf16_t*>(q),
                                          static_cast<hattn::bf16_t*>(k), pos0, B, S, tab,
                                          as_stream(stream)));
}

}  // extern "C"

namespace {

hattn_status kv_append_impl(const hattn_layer_cfg* cfg, const void* k_new, const void* v_new,
                            void* k_cache, void* v_cache, int32_t cap, const int32_t* pos0,
                            int32_t B, int32_t n, int32_t* slots_out, bool rope, void* stream) {
  hattn_status st = check_cfg(cfg);
  if (st != HATTN_OK) return st;
  if (B < 0 || n < 0 || cap < 1) return HATTN_ERR_SHAPE;
  if (cfg->kind == HATTN_SLIDING && cap != cfg->window) return HATTN_ERR_RANGE;
  const long long ntok = (long long)B * n;
  if (ntok == 0) return HATTN_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !pos0) return HATTN_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned4(pos0) || (slots_out && !aligned4(slots_out)))
    return HATTN_ERR_ALIGN;
  if (ntok * 256 > kMaxWorkItems) return HATTN_ERR_SHAPE;
  const hattn::RopeTable tab = rope_table(cfg);
  return hip_status(hattn::launch_kv_append(
      static_cast<const hattn::bf16_t*>(k_new), static_cast<const hattn::bf16_t*>(v_new),
      static_cast<hattn::bf16_t*>(k_cache), static_cast<hattn::bf16_t*>(v_cache), cap, pos0, B, n,
      cfg->kind == HATTN_SLIDING ? cfg->window : 0, slots_out, rope ? &tab : nullptr,
      as_stream(stream)));
}

}  // namespace

extern "C" {

hattn_status hattn_kv_append(const hattn_layer_cfg* cfg, const void* k_new, const void* v_new,
                             void* k_cache, void* v_cache, int32_t cap, const int32_t* pos0,
                             int32_t B, int32_t n, int32_t* slots_out, void* stream) {
  return kv_append_impl(cfg, k_new, v_new, k_cache, v_cache, cap, pos0, B, n, slots_out, false,
                        stream);
}

hattn_status hattn_kv_append_rope(const hattn_layer_cfg* cfg, const void* k_new,
                                  const void* v_new, void* k_cache, void* v_cache, int32_t cap,
                                  const int32_t* pos0, int32_t B, int32_t n, int32_t* slots_out,
                                  void* stream) {
  return kv_append_impl(cfg, k_new, v_new, k_cache, v_cache, cap, pos0, B, n, slots_out, true,
                        stream);
}

hattn_status hattn_prefill(const hattn_layer_cfg* cfg, const void* q, const void* k_cache,
                           const void* v_cache, int32_t cap, const int32_t* pos0, int32_t B,
                           int32_t Sq, const void* gate, void* out, float* lse, uint32_t flags,
                           void* stream) {
  hattn_status st = check_cfg(cfg);
  if (st != HATTN_OK) return st;
  if (B < 0 || Sq < 0 || cap < 1) return HATTN_ERR_SHAPE;
  if ((flags & ~(uint32_t)HATTN_ROPE_Q_FUSED) != 0) return HATTN_ERR_UNSUPPORTED;
  if ((long long)B * Sq == 0) return HATTN_OK;
  if (!q || !k_cache || !v_cache || !pos0 || !gate || !out) return HATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      !aligned2(gate) || !aligned4(pos0) || (lse && !aligned4(lse)))
    return HATTN_ERR_ALIGN;
  const long long nqb = ((long long)Sq + 31) / 32;
  const long long groups = (long long)B * hattn::kHkv * nqb + 8;
  if (groups * 256 > kMaxWorkItems || (long long)B * Sq >= (1LL << 31) ||
      (long long)B * cap >= (1LL << 40))
    return HATTN_ERR_SHAPE;
  const hattn::RopeTable tab = rope_table(cfg);
  return hip_status(hattn::launch_prefill(
      static_cast<const hattn::bf16_t*>(q), static_cast<const hattn::bf16_t*>(k_cache),
      static_cast<const hattn::bf16_t*>(v_cache), cap, pos0, B, Sq,
      static_cast<const hattn::bf16_t*>(gate), static_cast<hattn::bf16_t*>(out), lse,
      cfg->kind == HATTN_SLIDING ? cfg->window : 0, (flags & HATTN_ROPE_Q_FUSED) != 0, tab,
      scale_log2e(cfg), as_stream(stream)));
}

hattn_status hattn_prefill_ring(const hattn_layer_cfg* cfg, const void* q, const void* k_new,
                                const void* v_new, const void* k_ring, const void* v_ring,
                                const int32_t* pos0, int32_t B, int32_t Sq, const void* gate,
                                void* out, float* lse, uint32_t flags, void* stream) {
  hattn_status st = check_cfg(cfg);
  if (st != HATTN_OK) return st;
  if (cfg->kind != HATTN_SLIDING) return HATTN_ERR_UNSUPPORTED;
  if (B < 0 || Sq < 0) return HATTN_ERR_SHAPE;
  if ((flags & ~(uint32_t)HATTN_ROPE_Q_FUSED) != 0) return HATTN_ERR_UNSUPPORTED;
  if ((long long)B * Sq == 0) return HATTN_OK;
  if (!q || !k_new || !v_new || !k_ring || !v_ring || !pos0 || !gate || !out)
    return HATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_ring) ||
      !aligned16(v_ring) || !aligned16(out) || !aligned2(gate) || !aligned4(pos0) ||
      (lse && !aligned4(lse)))
    return HATTN_ERR_ALIGN;
  const long long nqb = ((long long)Sq + 31) / 32;
  const long long groups = (long long)B * hattn::kHkv * nqb + 8;
  if (groups * 256 > kMaxWorkItems || (long long)B * Sq >= (1LL << 31)) return HATTN_ERR_SHAPE;
  const hattn::RopeTable tab = rope_table(cfg);
  return hip_status(hattn::launch_prefill_ring(
      static_cast<const hattn::bf16_t*>(q), static_cast<const hattn::bf16_t*>(k_new),
      static_cast<const hattn::bf16_t*>(v_new), static_cast<const hattn::bf16_t*>(k_ring),
      static_cast<const hattn::bf16_t*>(v_ring), pos0, B, Sq,
      static_cast<const hattn::bf16_t*>(gate), static_cast<hattn::bf16_t*>(out), lse,
      cfg->window, (flags & HATTN_ROPE_Q_FUSED) != 0, tab, scale_log2e(cfg), as_stream(stream)));
}

hattn_status hattn_kv_append_fp8(const hattn_layer_cfg* cfg, const void* k_new,
                                 const void* v_new, void* k_cache, void* v_cache, float* k_scale,
                                 float* v_scale, int32_t cap, const int32_t* pos0, int32_t B,
                                 int32_t n, int32_t* slots_out, uint32_t flags, void* stream) {
  hattn_status st = check_cfg(cfg);
  if (st != HATTN_OK) return st;
  if (B < 0 || n < 0 || cap < 1) return HATTN_ERR_SHAPE;
  if ((flags & ~(uint32_t)HATTN_KV8_ROPE_K) != 0) return HATTN_ERR_UNSUPPORTED;
  if (cfg->kind == HATTN_SLIDING && cap != cfg->window) return HATTN_ERR_RANGE;
  const long long ntok = (long long)B * n;
  if (ntok == 0) return HATTN_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !k_scale || !v_scale || !pos0)
    return HATTN_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned4(k_scale) || !aligned4(v_scale) || !aligned4(pos0) ||
      (slots_out && !aligned4(slots_out)))
    return HATTN_ERR_ALIGN;
  if (ntok * 256 > kMaxWorkItems || (long long)B * cap >= (1LL << 40)) return HATTN_ERR_SHAPE;
  const hattn::RopeTable tab = rope_table(cfg);
  return hip_status(hattn::launch_kv_append_fp8(
      static_cast<const hattn::bf16_t*>(k_new), static_cast<const hattn::bf16_t*>(v_new),
      static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), k_scale, v_scale, cap, pos0,
      B, n, cfg->kind == HATTN_SLIDING ? cfg->window : 0, slots_out,
      (flags & HATTN_KV8_ROPE_K) ? &tab : nullptr, as_stream(stream)));
}

hattn_status hattn_decode_fp8(const hattn_layer_cfg* cfg, const void* q, const void* k_cache,
                              const void* v_cache, const float* k_scale, const float* v_scale,
                              int32_t cap, const int32_t* pos, int32_t B, const void* gate,
                              void* out, float* lse, void* workspace, size_t workspace_bytes,
                              uint32_t flags, void* stream) {
  hattn_status st = check_cfg(cfg);
  if (st != HATTN_OK) return st;
  if (B < 0 || cap < 1) return HATTN_ERR_SHAPE;
  if ((flags & ~(uint32_t)HATTN_ROPE_Q_FUSED) != 0) return HATTN_ERR_UNSUPPORTED;
  if (cfg->kind == HATTN_SLIDING && cap != cfg->window) return HATTN_ERR_RANGE;
  if (B == 0) return HATTN_OK;
  if (!q || !k_cache || !v_cache || !k_scale || !v_scale || !pos || !gate || !out)
    return HATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned4(k_scale) ||
      !aligned4(v_scale) || !aligned2(out) || !aligned2(gate) || !aligned4(pos) ||
      (lse && !aligned4(lse)))
    return HATTN_ERR_ALIGN;
  if (B > 65535 || (long long)B * cap >= (1LL << 40)) return HATTN_ERR_SHAPE;
  const hattn::DecodePlan plan = hattn::decode_plan(B, decode_max_keys(cfg, cap));
  const size_t need = hattn::decode_workspace_bytes(B, plan);
  if (workspace == nullptr || workspace_bytes < need) return HATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return HATTN_ERR_ALIGN;
  const hattn::RopeTable tab = rope_table(cfg);
  return hip_status(hattn::launch_decode_fp8(
      static_cast<const hattn::bf16_t*>(q), static_cast<const uint8_t*>(k_cache),
      static_cast<const uint8_t*>(v_cache), k_scale, v_scale, cap, pos, B,
      static_cast<const hattn::bf16_t*>(gate), static_cast<hattn::bf16_t*>(out), lse,
      cfg->kind == HATTN_SLIDING ? cfg->window : 0, (flags & HATTN_ROPE_Q_FUSED) != 0, tab,
      scale_log2e(cfg), plan, workspace, as_stream(stream)));
}

size_t hattn_decode_fp8_workspace_bytes(const hattn_layer_cfg* cfg, int32_t B, int32_t cap) {
  if (check_cfg(cfg) != HATTN_OK || B < 0 || cap < 1) return 0;
  if (cfg->kind == HATTN_SLIDING && cap != cfg->window) return 0;
  if (B == 0) return 0;
  return hattn::decode_workspace_bytes(B, hattn::decode_plan(B, decode_max_keys(cfg, cap)));
}

size_t hattn_decode_workspace_bytes(const hattn_layer_cfg* cfg, int32_t B, int32_t cap) {
  if (check_cfg(cfg) != HATTN_OK || B < 0 || cap < 1) return 0;
  if (cfg->kind == HATTN_SLIDING && cap != cfg->window) return 0;
  if (B == 0) return 0;
  return decode_need(cfg, B, cap);
}

}  // extern "C"

namespace {

// Checks of a decode call's arguments other than its workspace; *done is set when the
// call is empty (B == 0) and nothing is to be launched.
hattn_status check_decode(const hattn_layer_cfg* cfg, const void* q, const void* k_cache,
                          const void* v_cache, int32_t cap, const int32_t* pos, int32_t B,
                          const void* gate, void* out, float* lse, uint32_t flags, bool* done) {
  *done = false;
  hattn_status st = check_cfg(cfg);
  if (st != HATTN_OK) return st;
  if (B < 0 || cap < 1) return HATTN_ERR_SHAPE;
  if ((flags & ~(uint32_t)HATTN_ROPE_Q_FUSED) != 0) return HATTN_ERR_UNSUPPORTED;
  if (cfg->kind == HATTN_SLIDING && cap != cfg->window) return HATTN_ERR_RANGE;
  if (B == 0) {
    *done = true;
    return HATTN_OK;
  }
  if (!q || !k_cache || !v_cache || !pos || !gate || !out) return HATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned2(out) ||
      !aligned2(gate) || !aligned4(pos) || (lse && !aligned4(lse)))
    return HATTN_ERR_ALIGN;
  if (B > 65535 || (long long)B * cap >= (1LL << 40)) return HATTN_ERR_SHAPE;
  return HATTN_OK;
}

// The decode's launches on checked arguments and a workspace of at least decode_need bytes.
hattn_status decode_launch(const hattn_layer_cfg* cfg, const void* q, const void* k_cache,
                           const void* v_cache, int32_t cap, const int32_t* pos, int32_t B,
                           const void* gate, void* out, float* lse, void* workspace,
                           uint32_t flags, void* stream) {
  const hattn::DecodePlan plan = hattn::decode_plan(B, decode_max_keys(cfg, cap));
  const hattn::RopeTable tab = rope_table(cfg);
  if (cfg->kind == HATTN_SLIDING)
    return hip_status(hattn::launch_ring_decode(
        static_cast<const hattn::bf16_t*>(q), static_cast<const hattn::bf16_t*>(k_cache),
        static_cast<const hattn::bf16_t*>(v_cache), pos, B,
        static_cast<const hattn::bf16_t*>(gate), static_cast<hattn::bf16_t*>(out), lse,
        (flags & HATTN_ROPE_Q_FUSED) != 0, tab, scale_log2e(cfg), workspace, as_stream(stream)));
  return hip_status(hattn::launch_decode(
      static_cast<const hattn::bf16_t*>(q), static_cast<const hattn::bf16_t*>(k_cache),
      static_cast<const hattn::bf16_t*>(v_cache), cap, pos, B,
      static_cast<const hattn::bf16_t*>(gate), static_cast<hattn::bf16_t*>(out), lse,
      cfg->kind == HATTN_SLIDING ? cfg->window : 0, (flags & HATTN_ROPE_Q_FUSED) != 0, tab,
      scale_log2e(cfg), plan, workspace, as_stream(stream)));
}

// Scratch of hattn_decode_noalloc: the split partials (and a sliding ring split's partials
// and arrival counters) that hattn_decode keeps in the caller's workspace.  Each device
// the library runs on holds its own copy until the process ends.  Host code never passes
// this name to a kernel (on the host it is a stand-in, not a device address): it uses the
// address hipGetSymbolAddress returns for the current device, kept in g_scratch.
constexpr size_t kScratchBytes = HATTN_DECODE_NOALLOC_MAX_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The scratch array's address on the calling thread's current device, looked up on the
// first call on that device (with it current) and kept.
hattn_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return HATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return HATTN_OK;
}

}  // namespace

extern "C" {

hattn_status hattn_decode(const hattn_layer_cfg* cfg, const void* q, const void* k_cache,
                          const void* v_cache, int32_t cap, const int32_t* pos, int32_t B,
                          const void* gate, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, uint32_t flags, void* stream) {
  bool done = false;
  const hattn_status st =
      check_decode(cfg, q, k_cache, v_cache, cap, pos, B, gate, out, lse, flags, &done);
  if (st != HATTN_OK || done) return st;
  const size_t need = decode_need(cfg, B, cap);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return HATTN_ERR_WORKSPACE;
  if (workspace != nullptr && !aligned16(workspace)) return HATTN_ERR_ALIGN;
  return decode_launch(cfg, q, k_cache, v_cache, cap, pos, B, gate, out, lse, workspace, flags,
                       stream);
}

hattn_status hattn_decode_noalloc(const hattn_layer_cfg* cfg, const void* q, const void* k_cache,
                                  const void* v_cache, int32_t cap, const int32_t* pos, int32_t B,
                                  const void* gate, void* out, float* lse, uint32_t flags,
                                  void* stream) {
  bool done = false;
  hattn_status st =
      check_decode(cfg, q, k_cache, v_cache, cap, pos, B, gate, out, lse, flags, &done);
  if (st != HATTN_OK || done) return st;
  if (decode_need(cfg, B, cap) > kScratchBytes) return HATTN_ERR_SCRATCH;
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != HATTN_OK) return st;
  return decode_launch(cfg, q, k_cache, v_cache, cap, pos, B, gate, out, lse, ws, flags, stream);
}

hattn_status hattn_qkv_proj(const void* x, int32_t T, const void* w_qkv, const void* w_gate,
                            void* q, void* k, void* v, void* gate, void* stream) {
  if (T < 0) return HATTN_ERR_SHAPE;
  if (T == 0) return HATTN_OK;
  if (!x || !w_qkv || !w_gate || !q || !k || !v || !gate) return HATTN_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_qkv) || !aligned16(w_gate) || !aligned16(q) ||
      !aligned16(k) || !aligned16(v) || !aligned16(gate))
    return HATTN_ERR_ALIGN;
  if ((long long)T > 65535LL * 128) return HATTN_ERR_SHAPE;
  return hip_status(hattn::launch_qkv_proj(
      static_cast<const hattn::bf16_t*>(x), T, static_cast<const hattn::bf16_t*>(w_qkv),
      static_cast<const hattn::bf16_t*>(w_gate), static_cast<hattn::bf16_t*>(q),
      static_cast<hattn::bf16_t*>(k), static_cast<hattn::bf16_t*>(v),
      static_cast<hattn::bf16_t*>(gate), as_stream(stream)));
}

hattn_status hattn_o_proj(const void* attn, int32_t T, const void* w_o, void* y, void* stream) {
  if (T < 0) return HATTN_ERR_SHAPE;
  if (T == 0) return HATTN_OK;
  if (!attn || !w_o || !y) return HATTN_ERR_NULL;
  if (!aligned16(attn) || !aligned16(w_o) || !aligned16(y)) return HATTN_ERR_ALIGN;
  if ((long long)T > 65535LL * 128) return HATTN_ERR_SHAPE;
  return hip_status(hattn::launch_o_proj(static_cast<const hattn::bf16_t*>(attn), T,
                                         static_cast<const hattn::bf16_t*>(w_o),
                                         static_cast<hattn::bf16_t*>(y), as_stream(stream)));
}

const char* hattn_status_string(hattn_status status) {
  switch (status) {
    case HATTN_OK: return "ok";
    case HATTN_ERR_NULL: return "a required pointer is NULL";
    case HATTN_ERR_SHAPE: return "invalid or too large size";
    case HATTN_ERR_UNSUPPORTED: return "unsupported layer configuration or flag";
    case HATTN_ERR_RANGE: return "cache capacity or window rule broken";
    case HATTN_ERR_ALIGN: return "tensor pointer not aligned";
    case HATTN_ERR_WORKSPACE: return "decode workspace missing or too small";
    case HATTN_ERR_HIP: return "HIP launch failed";
    case HATTN_ERR_SCRATCH:
      return "decode needs more scratch than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

int32_t hattn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
