/*
 * hattn -- hybrid GQA attention layer for AMD Instinct MI355X (gfx950).
 *
 * One attention layer of the Spark-X2.5 / X2.6-4B model family: sliding-window layers
 * (window 512, RoPE base 1e4 over all 256 dims) and full-causal layers (RoPE base 5e6
 * over dims 0..63, dims 64..255 unrotated), both GQA with 16 query heads over 4 KV heads,
 * head_dim 256, softmax scale 1/16 and a per-head sigmoid output gate.
 *
 * Sources (web pages, cited by title and section):
 *   [T1] "How a million tokens fit into a 4B model: Spark X2.5's long-context
 *        architecture and its memory trade-offs" (hotelren.com)
 *   [T2] "No high-VRAM card needed: a 4B model takes on a million-token context"
 *        (163.com)
 *   [T3] "Spark-X2.6-4B-Base hybrid attention architecture" (lqnn.cn)
 *
 * Conventions for every call:
 *   - All tensors are caller-owned DEVICE memory; the library allocates nothing and keeps
 *     no state between calls except a thread-local last HIP error code.
 *   - Activations are bf16 (raw 16-bit words), row-major "BSHD":
 *       q, out     [B, S, 16, 256]     gate [B, S, 16]     lse [B, S, 16] fp32
 *       k, v       [B, S, 4, 256]      caches [B, cap, 4, 256]
 *     The element (b, s, h, d) sits at ((b*S + s)*H + h)*256 + d.
 *   - Position arrays are int32 in device memory and are read by the kernels.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call
 *     returns; results are valid once the stream has reached that point.
 *   - Arguments are validated on the host before any launch.  A call with an empty size
 *     (no tokens or no sequences) returns HATTN_OK without looking at its pointers
 *     (empty torch tensors carry NULL data pointers).  A non-OK status means
 *     nothing was enqueued, except HATTN_ERR_HIP (a launch failed; see
 *     hattn_last_hip_error).  No C++ exception crosses this interface.
 *   - Device-side range guards: a key index outside [0, cap) is never read and a cache
 *     slot outside [0, cap) is never written, whatever the position arrays hold.
 *   - Calls are reentrant; calls on different streams may run concurrently as long as
 *     they do not write the same buffers.
 */
#ifndef HATTN_H_
#define HATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t hattn_status;
enum {
  HATTN_OK = 0,
  HATTN_ERR_NULL = 1,        /* a required pointer is NULL                             */
  HATTN_ERR_SHAPE = 2,       /* a size is negative or too large for 32-bit indexing     */
  HATTN_ERR_UNSUPPORTED = 3, /* heads / head_dim / rot_dim / window not the model's     */
  HATTN_ERR_RANGE = 4,       /* cap, window or position-range rule broken               */
  HATTN_ERR_ALIGN = 5,       /* a tensor pointer is not 16-byte aligned                 */
  HATTN_ERR_WORKSPACE = 6,   /* decode workspace NULL or smaller than required          */
  HATTN_ERR_HIP = 7,         /* a HIP launch failed; hattn_last_hip_error() has the code */
  HATTN_ERR_SCRATCH = 8      /* hattn_decode_noalloc: the call needs more scratch than
                                HATTN_DECODE_NOALLOC_MAX_BYTES                        */
};

/* Layer kinds.  [T1] "Hybrid attention: only one layer in four gets the full view";
 * [T2] "27 sliding-window layers plus 9 global layers". */
enum { HATTN_SLIDING = 0, HATTN_FULL = 1 };

/* hattn_prefill flag: q is given unrotated and the kernel applies RoPE to it in its
 * prologue (otherwise q must already be rotated). */
enum { HATTN_ROPE_Q_FUSED = 1u };

/* Per-layer configuration.  Only the model's values are supported:
 *   n_q_heads 16, n_kv_heads 4, head_dim 256, softmax_scale 1/16;
 *   sliding: window 512, rot_dim 256, rope_theta 1e4;
 *   full:    window 0,   rot_dim 64,  rope_theta 5e6.
 * [T1] "GQA, fused projection and output gating" (heads, head_dim); [T1] "Per-layer RoPE
 * and the local/global split" and [T3] "Global attention + 5M-base RoPE" (theta, the
 * rotary fraction 0.25 = 64 dims); [T3] "Sliding window 512". */
typedef struct hattn_layer_cfg {
  int32_t kind;        /* HATTN_SLIDING or HATTN_FULL                       */
  int32_t n_q_heads;   /* 16                                                */
  int32_t n_kv_heads;  /* 4                                                 */
  int32_t head_dim;    /* 256                                               */
  int32_t window;      /* 512 for sliding, 0 for full                       */
  int32_t rot_dim;     /* leading dims that rotate: 256 sliding, 64 full    */
  double rope_theta;   /* 1e4 sliding, 5e6 full                             */
  float softmax_scale; /* 1/16                                              */
  int32_t reserved;    /* must be 0                                         */
} hattn_layer_cfg;

/* Fill *out with the preset for `kind`.  HATTN_ERR_NULL / HATTN_ERR_UNSUPPORTED. */
hattn_status hattn_cfg_preset(int32_t kind, hattn_layer_cfg* out);

/* RoPE, in place, on q [B,S,16,256] and/or k [B,S,4,256] (either may be NULL, not both).
 * Token s of sequence b sits at position pos0[b] + s (pos0: int32 [B], device); positions
 * are int32, so pos0[b] + S - 1 <= 2^31 - 1 (checked nowhere: pos0 lives on the device).
 * Pair (i, i + r/2), i < r/2 with r = rot_dim, turns by angle
 *   a = float32( float32(pos) * float32(theta ** (-2 i / r)) )
 * (rotate-half pairing); dims r..255 are neither read nor written.  fp32 arithmetic,
 * results rounded to bf16 (nearest-even).
 * [T1] "Per-layer RoPE and the local/global split" (rope_parameters per layer type,
 * compute_rope_cos_sin / apply_rotary_pos_emb); [T3] "Global attention + 5M-base RoPE". */
hattn_status hattn_rope_qk(const hattn_layer_cfg* cfg, void* q, void* k, const int32_t* pos0,
                           int32_t B, int32_t S, void* stream);

/* Copy n rotated tokens per sequence, k_new / v_new [B,n,4,256], into the caches
 * k_cache / v_cache [B,cap,4,256].  Token t of sequence b has position p = pos0[b] + t,
 * an int32: pos0[b] + n - 1 <= 2^31 - 1 (a larger value wraps negative and is skipped).
 *   full:    slot = p; tokens with p < 0 or p >= cap are skipped (slot reported -1).
 *   sliding: cap must equal cfg->window (the ring); slot = p mod window; when n > window
 *            only the last `window` tokens are written (a later token would overwrite
 *            an earlier one in the same slot), but every token's slot is reported.
 * slots_out: int32 [B,n] device, may be NULL.
 * [T2] "The real bottleneck of a million-token context" (sliding layers keep only the
 * most recent 512 tokens' keys and values, full layers keep them all); [T1] "Doing the
 * arithmetic first" (4096 bytes per token per layer). */
hattn_status hattn_kv_append(const hattn_layer_cfg* cfg, const void* k_new, const void* v_new,
                             void* k_cache, void* v_cache, int32_t cap, const int32_t* pos0,
                             int32_t B, int32_t n, int32_t* slots_out, void* stream);

/* hattn_kv_append with the RoPE of the keys fused in: k_new [B,n,4,256] holds UNROTATED
 * keys, and each is rotated by its position (the arithmetic of hattn_rope_qk, bit for bit)
 * as it is written to the cache; k_new itself is not modified, so a captured sequence of
 * calls can be replayed.  Slots, ring rules, status codes and v_new as in hattn_kv_append.
 * [T1] "Per-layer RoPE and the local/global split"; [T2] "The real bottleneck of a
 * million-token context". */
hattn_status hattn_kv_append_rope(const hattn_layer_cfg* cfg, const void* k_new,
                                  const void* v_new, void* k_cache, void* v_cache, int32_t cap,
                                  const int32_t* pos0, int32_t B, int32_t n, int32_t* slots_out,
                                  void* stream);

/* Prefill attention for Sq query tokens per sequence.
 *   q [B,Sq,16,256] (unrotated if flags & HATTN_ROPE_Q_FUSED, else rotated);
 *   k_cache / v_cache [B,cap,4,256]: rotated keys and values indexed by absolute position
 *     (row j holds the token at position j), for both layer kinds;
 *   query i of sequence b sits at p = pos0[b] + i and sees the keys at positions
 *     full:    0 .. p          sliding: max(0, p - window + 1) .. p
 *     clipped to [0, cap) (callers keep pos0[b] + Sq <= cap);
 *   gate [B,Sq,16] bf16 logits; out [B,Sq,16,256] bf16; lse [B,Sq,16] fp32 or NULL.
 * Per (b, i, h) with kv head h/4:  s_j = (q . k_j) * softmax_scale,
 *   out = bf16( sigmoid(gate) * sum_j softmax(s)_j v_j ),  lse = ln sum_j exp(s_j).
 * A row with no visible key gets out = 0 and lse = -inf.
 * [T1] "Hybrid attention" (create_causal_mask / create_sliding_window_causal_mask per layer
 * type); [T1] "GQA, fused projection and output gating" (16 query heads share 4 KV heads;
 * gate = sigmoid(gate_score.float()), attn_output * gate); [T2] "Grouped-query attention". */
hattn_status hattn_prefill(const hattn_layer_cfg* cfg, const void* q, const void* k_cache,
                           const void* v_cache, int32_t cap, const int32_t* pos0, int32_t B,
                           int32_t Sq, const void* gate, void* out, float* lse, uint32_t flags,
                           void* stream);

/* Sliding-layer prefill of a chunk that continues a ring cache (cfg->kind must be
 * HATTN_SLIDING, else HATTN_ERR_UNSUPPORTED).  Sequence b's chunk holds Sq tokens at
 * positions p = pos0[b] + i, i < Sq:
 *   q [B,Sq,16,256] (unrotated if flags & HATTN_ROPE_Q_FUSED, else rotated), gate [B,Sq,16];
 *   k_new / v_new [B,Sq,4,256]: the chunk's rotated keys and values;
 *   k_ring / v_ring [B,512,4,256]: the ring as hattn_kv_append leaves it after positions
 *     0 .. pos0[b] - 1 were appended in order (slot = position mod 512).  Slots that no
 *     position has reached yet (pos0[b] < 512) are never read.
 * Query i sees positions max(0, p - 511) .. p: those below pos0[b] from the ring, the rest
 * from k_new / v_new.  out [B,Sq,16,256] bf16, lse [B,Sq,16] fp32 or NULL; same arithmetic
 * and empty-row rule as hattn_prefill.  The ring is only read: append the chunk with
 * hattn_kv_append after this call (appending first would overwrite keys that the chunk's
 * earlier rows still see).  pos0[b] >= 0 and pos0[b] + Sq <= 2^31 - 1; the kernel clamps
 * larger positions and never reads outside the given buffers.
 * [T2] "The real bottleneck of a million-token context" (sliding layers keep only the last
 * 512 tokens' keys and values); [T3] "Sliding window 512"; [T1] "Hybrid attention". */
hattn_status hattn_prefill_ring(const hattn_layer_cfg* cfg, const void* q, const void* k_new,
                                const void* v_new, const void* k_ring, const void* v_ring,
                                const int32_t* pos0, int32_t B, int32_t Sq, const void* gate,
                                void* out, float* lse, uint32_t flags, void* stream);

/* Bytes of device workspace hattn_decode needs for B sequences and this cache capacity:
 * a full layer's split-KV partial results; a sliding layer's ring-split partials and
 * arrival counters.  0 for an invalid configuration. */
size_t hattn_decode_workspace_bytes(const hattn_layer_cfg* cfg, int32_t B, int32_t cap);

/* Single-token decode.  q [B,1,16,256] (rotated unless flags & HATTN_ROPE_Q_FUSED),
 * gate [B,1,16], out [B,1,16,256], lse [B,1,16] fp32 or NULL; pos: int32 [B] device,
 * the new token's position, whose key/value must already be in the cache.
 *   full:    k_cache / v_cache [B,cap,4,256], keys at rows 0 .. pos[b] (clipped to cap);
 *   sliding: the ring [B,window,4,256] (cap must equal window); the first
 *            min(pos[b] + 1, window) slots are valid (the ring is filled in position
 *            order from position 0), and every valid slot is visible.  All 512 slots
 *            are read (their loads go out before the position is known); the others
 *            may hold anything, NaN included, and never reach the result.
 * Same arithmetic as hattn_prefill.  The key range is split into chunks whose partial
 * (max, sum, output) triples are merged by log-sum-exp in a second kernel.  A sliding
 * layer runs as one kernel instead: 8 workgroups per (sequence, KV head) for B <= 8, 4
 * above, each take an equal share of the 512 ring slots, and the last of them to finish
 * merges their partials; the arrival counters live in the workspace and the call clears
 * them first (a small kernel ahead of it on `stream`), so calls that share a workspace
 * must be ordered (one stream); they race otherwise.
 * workspace: device, at least hattn_decode_workspace_bytes(cfg, B, cap) bytes (16-byte
 * aligned).
 * B <= 65535 (one grid row per sequence), else HATTN_ERR_SHAPE.
 * [T2] "The real bottleneck of a million-token context" (the ring keeps the last 512
 * tokens); [T1] "GQA, fused projection and output gating". */
hattn_status hattn_decode(const hattn_layer_cfg* cfg, const void* q, const void* k_cache,
                          const void* v_cache, int32_t cap, const int32_t* pos, int32_t B,
                          const void* gate, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, uint32_t flags, void* stream);

/* hattn_decode for callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc -- and so cannot pass a
 * workspace.  Arguments, layouts, arithmetic and results as hattn_decode (the same kernels
 * and split plan); the partials and counters that hattn_decode keeps in the caller's
 * workspace go to a static device array of HATTN_DECODE_NOALLOC_MAX_BYTES bytes instead,
 * which each GPU the library runs on holds until the process ends.  The call allocates
 * nothing (no hipMalloc, no library routine that allocates).  Its first call on a device
 * looks up that device's copy of the array (the calling thread's current device, which
 * must be the device of `stream` and of the buffers) and keeps its address.
 *   HATTN_ERR_SCRATCH: hattn_decode_workspace_bytes(cfg, B, cap) exceeds
 *     HATTN_DECODE_NOALLOC_MAX_BYTES (a full layer at B up to about 2000 fits, a sliding
 *     layer at B up to 507); nothing is
 *     enqueued.  Other errors as hattn_decode.
 * Every call on one GPU shares that GPU's array and leaves its contents behind; each call
 * clears what must start at zero.  Calls that overlap on one GPU (on different streams, or
 * from different host threads without ordering) race on the array and give wrong
 * results: order them on one stream. */
#define HATTN_DECODE_NOALLOC_MAX_BYTES ((size_t)32 << 20)
hattn_status hattn_decode_noalloc(const hattn_layer_cfg* cfg, const void* q, const void* k_cache,
                                  const void* v_cache, int32_t cap, const int32_t* pos, int32_t B,
                                  const void* gate, void* out, float* lse, uint32_t flags,
                                  void* stream);

/* ---- 8-bit KV cache ------------------------------------------------------------------
 * The library's own 8-bit cache format (for the quantized KV cache the pages' 1M
 * deployment uses: [T5] "Why fitting a 1M context into a 4B dense model deserves its own
 * discussion", §3.2 "Deployment steps and key parameters"):
 *   k_cache / v_cache [B,cap,4,256] uint8 OCP FP8 E4M3 codes (sign, 4 exponent bits with
 *     bias 7, 3 mantissa bits; 0x7F / 0xFF NaN; largest finite 448);
 *   k_scale / v_scale [B,4,cap] fp32, one per (token, KV head) -- head-major so a head's
 *     scales of consecutive tokens are contiguous.
 * A stored row x (256 values of one head, the bf16 a 16-bit cache would hold) becomes
 *   scale = fp32(amax|x| / 448),  code_d = E4M3_RNE(clamp(fp32(x_d / scale), -448, 448))
 * (all codes 0 and scale 0 for an all-zero row); its value is code_value * scale.
 * 2080 bytes per token per layer instead of 4096. */

/* hattn_kv_append_fp8 flag: k_new is unrotated; rotate it by position first (the bits of
 * hattn_rope_qk), then quantize.  Without it k_new must already be rotated. */
enum { HATTN_KV8_ROPE_K = 1u };

/* Quantize and append n tokens per sequence (positions pos0[b] + t) into an 8-bit cache;
 * k_new / v_new [B,n,4,256] bf16 are only read.  Slots, ring rules, slots_out and status
 * codes as hattn_kv_append; the scales of a written slot are overwritten with the codes. */
hattn_status hattn_kv_append_fp8(const hattn_layer_cfg* cfg, const void* k_new,
                                 const void* v_new, void* k_cache, void* v_cache, float* k_scale,
                                 float* v_scale, int32_t cap, const int32_t* pos0, int32_t B,
                                 int32_t n, int32_t* slots_out, uint32_t flags, void* stream);

/* hattn_decode over an 8-bit cache: the attention of the dequantized keys and values (the
 * key scale multiplies its score, the value scale its probability).  Arguments, flags and
 * errors as hattn_decode; the workspace (16-byte aligned) holds the split-KV partials for
 * both layer kinds: at least hattn_decode_fp8_workspace_bytes(cfg, B, cap) bytes. */
size_t hattn_decode_fp8_workspace_bytes(const hattn_layer_cfg* cfg, int32_t B, int32_t cap);
hattn_status hattn_decode_fp8(const hattn_layer_cfg* cfg, const void* q, const void* k_cache,
                              const void* v_cache, const float* k_scale, const float* v_scale,
                              int32_t cap, const int32_t* pos, int32_t B, const void* gate,
                              void* out, float* lse, void* workspace, size_t workspace_bytes,
                              uint32_t flags, void* stream);

/* ---- Whole-model driver ------------------------------------------------------------
 * The model's layers follow one schedule: layer l is full-causal iff l % 4 == 3, every
 * other layer sliding-window (36 layers: 9 full, 27 sliding).  [T1] "Hybrid attention:
 * only one layer in four gets the full view"; [T2] "27 sliding-window layers plus 9 global
 * layers"; [T3] "36-layer hybrid layout". */

/* HATTN_FULL or HATTN_SLIDING for layer index `layer` (-1 if negative). */
int32_t hattn_model_layer_kind(int32_t layer);

/* KV-cache bytes of the schedule for B sequences: a full layer keeps cap tokens, a sliding
 * layer its 512-slot ring, each token 4096 bytes (K and V, 4 heads x 256 dims x bf16).
 * per_layer (host, n_layers entries) may be NULL; total (host) is required.
 * HATTN_ERR_SHAPE unless 1 <= n_layers <= 4096, B >= 0, cap >= 512.
 * [T1] "Doing the arithmetic first" (4096 bytes per token per layer). */
hattn_status hattn_model_kv_bytes(int32_t n_layers, int32_t B, int32_t cap, size_t* per_layer,
                                  size_t* total);

/* One layer's buffers for a driver call (all device memory, layouts as above):
 *   q [B,S,16,256], k / v [B,S,4,256] (q and k UNROTATED), gate [B,S,16];
 *   k_cache / v_cache: full layers [B,cap,4,256] (position-indexed), sliding layers the
 *     ring [B,512,4,256];  out [B,S,16,256];  lse [B,S,16] fp32 or NULL.
 * S is 1 for hattn_model_decode and Sq for hattn_model_prefill.  Inputs are only read. */
typedef struct hattn_layer_io {
  const void* q;
  const void* k;
  const void* v;
  const void* gate;
  void* k_cache;
  void* v_cache;
  void* out;
  float* lse;
} hattn_layer_io;

/* Device workspace hattn_model_decode needs (0 for invalid sizes): the full layers' split
 * partials and the sliding layers' ring partials and per-head counters.  Its
 * contents between calls do not matter: each call clears the counters (with a kernel) before
 * its first sliding layer. */
size_t hattn_model_decode_workspace_bytes(int32_t n_layers, int32_t B, int32_t cap);

/* One decode step of every layer, in layer order, on `stream`: for each layer the new
 * token at pos[b] (int32 [B], device) is rotated and appended (hattn_kv_append_rope) and
 * attended (hattn_decode with HATTN_ROPE_Q_FUSED); a sliding layer does both in one launch
 * (the same arithmetic).  layers: host array of n_layers.  workspace: device, 16-byte
 * aligned, at least hattn_model_decode_workspace_bytes(n_layers, B, cap) bytes; calls
 * that overlap on one workspace race.
 * Nothing is allocated and no input is modified, so a captured step replays exactly.
 * All pointers are checked before anything is enqueued; a later non-OK status can only
 * be HATTN_ERR_HIP.  Errors: those of the per-layer calls, HATTN_ERR_WORKSPACE, and
 * HATTN_ERR_SHAPE unless 1 <= n_layers <= 4096, 0 <= B <= 65535, cap >= 512. */
hattn_status hattn_model_decode(const hattn_layer_io* layers, int32_t n_layers, int32_t cap,
                                const int32_t* pos, int32_t B, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Device workspace hattn_model_prefill needs: one sliding layer's rotated chunk keys. */
size_t hattn_model_prefill_workspace_bytes(int32_t n_layers, int32_t B, int32_t Sq);

/* One prefill chunk of Sq tokens per sequence (positions pos0[b] ..) through every layer:
 *   full:    hattn_kv_append_rope into the cache, then hattn_prefill over it;
 *   sliding: the chunk's keys are rotated into the workspace, attended together with the
 *            ring (hattn_prefill_ring), then appended to the ring.
 * Chunks must arrive in position order, each after the previous one's call.
 * HATTN_ERR_SHAPE unless 1 <= n_layers <= 4096, 0 <= B <= 65535, cap >= 512, Sq >= 0. */
hattn_status hattn_model_prefill(const hattn_layer_io* layers, int32_t n_layers, int32_t cap,
                                 const int32_t* pos0, int32_t B, int32_t Sq, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ---- Projections around the layer ------------------------------------------------
 * [T1] "GQA, fused projection and output gating": one linear layer q_k_v_proj of width
 * q_dim + 2 kv_dim whose output is sliced in that order into q, k and v, and g_proj
 * giving one gate score per head; [T4] parameter table (hidden_size 2560) and its
 * quantization section (o_proj).  Weights in the linear-layer layout [out, in], bf16, no
 * bias; fp32 accumulation, outputs rounded to bf16 (nearest-even).  All device memory,
 * 16-byte aligned; T = 0 returns HATTN_OK without looking at the pointers. */

/* x [T,2560] -> q [T,16,256] (unrotated), k [T,4,256] (unrotated), v [T,4,256] and gate
 * logits [T,16], the layouts the attention calls take; w_qkv [6144,2560] (rows 0..4095 q,
 * 4096..5119 k, 5120..6143 v), w_gate [16,2560]. */
hattn_status hattn_qkv_proj(const void* x, int32_t T, const void* w_qkv, const void* w_gate,
                            void* q, void* k, void* v, void* gate, void* stream);

/* attn [T,16,256] (gated head outputs, heads concatenated) -> y [T,2560] with w_o
 * [2560,4096]. */
hattn_status hattn_o_proj(const void* attn, int32_t T, const void* w_o, void* y, void* stream);

/* Static description of a status code. */
const char* hattn_status_string(hattn_status status);

/* The hipError_t of the last HATTN_ERR_HIP on the calling thread (0 if none). */
int32_t hattn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HATTN_H_ */
