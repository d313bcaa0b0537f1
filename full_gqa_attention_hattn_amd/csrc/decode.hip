// Single-token decode for one hybrid-attention layer on CDNA4 (gfx950): split-KV partials
// followed by a log-sum-exp combine.
//
// Full layers read keys 0..pos of a position-indexed cache; sliding layers read the
// 512-slot ring (slot = position mod 512), every valid slot being inside the window.
// [T2] "The real bottleneck of a million-token context" (full layers keep the whole
// history, sliding layers only the last 512 tokens); [T1] "GQA, fused projection and
// output gating" (4 query heads per KV head; sigmoid head gate).
//
// Phase 1 (decode_split_kernel): grid (chunks, B); wave w of a workgroup handles KV head w
// over the chunk's keys, so a workgroup streams whole 2 KiB cache rows (4 heads x 512 B).
// Per 32-key step a wave computes S^T = K . Q^T for its 4 query heads on
// v_mfma_f32_16x16x32_bf16 (K rows feed the MFMA straight from global memory; columns
// 4..15 of Q^T are zero), runs the online softmax, and accumulates P.V on the VALU with the
// probabilities broadcast through LDS: two keys at a time with v_dot2_f32_bf16 (the same
// dim of both keys permuted into one bf16 pair, the probabilities rounded to bf16).  The
// reference max moves only when a step beats it by more than 2^8, so O is rarely
// rescaled.  It writes a partial (reference max, sum, o[4][256]) per (b, kv head, chunk).
// Phase 2 (decode_combine_kernel): per (b, query head, 32-dim slice), merges the chunk
// partials by log-sum-exp, applies 1/l and the sigmoid gate, stores bf16 (and the LSE).
#include "hattn_device.h"
#include "hattn_launch.h"

namespace hattn {

namespace {

constexpr int kStep = 32;  // keys per wave step
constexpr float kRescaleLog2 = 8.f;  // move the reference max only when beaten by 2^8
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void wave_lds_fence() {
  // LDS traffic of one wave is processed in order; this keeps the compiler from moving the
  // probability stores and loads across each other.
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// Operands of one 32-key step of a wave: K rows (MFMA view) and V rows (PV view).
struct StepRegs {
  bf16x8 kf[2][8];
  uint4 vv[16];
};

// Issue this lane's loads of the step at keys k0 .. k0 + 31 (of [.., k_end)) of the KV
// head whose cache rows (4 heads x 256 dims) start at kb / vb.
__device__ __forceinline__ void load_step(StepRegs& r, const bf16_t* kb, const bf16_t* vb, int k0,
                                          int k_end, int lane) {
  constexpr long long rs = kHkv * kD;
  const int n16 = lane & 15, g = lane >> 4;    // MFMA view: column (head) and k-group
  const int half = lane >> 5, dg = lane & 31;  // PV view: key parity and 8-dim group
  // Keys past k_end read row k_end - 1 instead (their scores are masked to -inf, so those
  // values meet a zero probability): unconditional loads the compiler can count, so the
  // QK chain waits only for K while V is still in flight.
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int key = min(k0 + 16 * blk + n16, k_end - 1);
    const bf16_t* kr = kb + (long long)key * rs + 8 * g;
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) r.kf[blk][dc] = *reinterpret_cast<const bf16x8*>(kr + 32 * dc);
  }
#pragma unroll
  for (int kp = 0; kp < 16; ++kp) {
    const int key = min(k0 + 2 * kp + half, k_end - 1);
    r.vv[kp] = *reinterpret_cast<const uint4*>(vb + (long long)key * rs + 8 * dg);
  }
}

// One 32-key step on loaded operands: S^T = K . Q^T on MFMA, the online softmax and P.V on
// the VALU, the probabilities going through this wave's slice `pl` of LDS.
__device__ __forceinline__ void compute_step(const StepRegs& r, const bf16x8 (&qf)[8], int k0,
                                             int k_end, float sl2, float (*pl)[4], int lane,
                                             float& m_run, float& l_run, float (&o)[kGroup][8]) {
  const int n16 = lane & 15, g = lane >> 4;
  const int half = lane >> 5;
  const bool qlane = n16 < kGroup;
  f32x4 s[2] = {f32x4{}, f32x4{}};
#pragma unroll
  for (int dc = 0; dc < 8; ++dc) {
    s[0] = mfma16(r.kf[0][dc], qf[dc], s[0]);
    s[1] = mfma16(r.kf[1][dc], qf[dc], s[1]);
  }
  // s[blk][j] = score of key k0 + 16 blk + 4g + j for head column n16.
  float mloc = -INFINITY;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = k0 + 16 * blk + 4 * g + j;
      const float v = key < k_end ? s[blk][j] * sl2 : -INFINITY;
      s[blk][j] = v;
      mloc = fmaxf(mloc, v);
    }
  mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
  // The reference max moves only when a step beats it by more than 2^8 (or on the first
  // visible key): probabilities stay below 256, and O is rescaled on those steps only.
  const bool bump = mloc > m_run + kRescaleLog2 || (m_run == -INFINITY && mloc != -INFINITY);
  if (__any(bump)) {
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
    l_run *= alpha;
    m_run = m_new;
    // Per-head factors live in lanes 0..3 (column = head, k-group 0).
    const float a0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 0));
    const float a1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 1));
    const float a2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 2));
    const float a3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 3));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[0][e] *= a0;
      o[1][e] *= a1;
      o[2][e] *= a2;
      o[3][e] *= a3;
    }
  }
  const float m_use = m_run == -INFINITY ? 0.f : m_run;
  float rsum = 0.f;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float pj = fast_exp2(s[blk][j] - m_use);
      s[blk][j] = pj;
      rsum += pj;
    }
  l_run += rsum;

  if (qlane) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int j = 0; j < 4; ++j) pl[16 * blk + 4 * g + j][n16] = s[blk][j];
  }
  wave_lds_fence();
  // Keys a = 2kp + half and b = a + 2 share a lane: one permute gathers the same dim of
  // both into a bf16 pair, and one dot2 adds p_a v_a + p_b v_b (probabilities in bf16).
#pragma unroll
  for (int kp = 0; kp < 16; kp += 2) {
    const f32x4 pa = *reinterpret_cast<const f32x4*>(&pl[2 * kp + half][0]);
    const f32x4 pb = *reinterpret_cast<const f32x4*>(&pl[2 * kp + 2 + half][0]);
    bf16x2 pp[kGroup];
#pragma unroll
    for (int hl = 0; hl < kGroup; ++hl) pp[hl] = __builtin_bit_cast(bf16x2, pack_bf16x2(pa[hl], pb[hl]));
    const uint32_t* va = reinterpret_cast<const uint32_t*>(&r.vv[kp]);
    const uint32_t* vb2 = reinterpret_cast<const uint32_t*>(&r.vv[kp + 1]);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const bf16x2 d0 = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(vb2[w], va[w], 0x05040100u));
      const bf16x2 d1 = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(vb2[w], va[w], 0x07060302u));
#pragma unroll
      for (int hl = 0; hl < kGroup; ++hl) {
        o[hl][2 * w] = __builtin_amdgcn_fdot2_f32_bf16(d0, pp[hl], o[hl][2 * w], false);
        o[hl][2 * w + 1] = __builtin_amdgcn_fdot2_f32_bf16(d1, pp[hl], o[hl][2 * w + 1], false);
      }
    }
  }
  wave_lds_fence();
}

// One wave's pass over keys [k_begin, k_end) of its KV head, one 32-key step at a time.
// Leaves this lane's share of the partial (reference max, sum, o[head][8 dims]).
__device__ __forceinline__ void attend_keys(const bf16x8 (&qf)[8], const bf16_t* kb,
                                            const bf16_t* vb, int k_begin, int k_end, float sl2,
                                            float (*pl)[4], int lane, float& m_run, float& l_run,
                                            float (&o)[kGroup][8]) {
  for (int k0 = k_begin; k0 < k_end; k0 += kStep) {
    StepRegs r;
    load_step(r, kb, vb, k0, k_end, lane);
    compute_step(r, qf, k0, k_end, sl2, pl, lane, m_run, l_run, o);
  }
}

template <bool kSliding>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
    int cap, const int* __restrict__ pos, int window, int chunk, int nchunks,
    float* __restrict__ ws_o, float* __restrict__ ws_ml, int rope_q, RopeTable tab, float sl2) {
  constexpr int kNdc = kSliding ? 4 : 1;  // Q fragments (32 dims each) in the first rotary half
  __shared__ __attribute__((aligned(16))) float p_lds[kHkv][kStep][4];

  const int c = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, kvh = tid >> 6;
  const int n16 = lane & 15, g = lane >> 4;    // MFMA view: column (head) and k-group
  const int half = lane >> 5, dg = lane & 31;  // PV view: key parity and 8-dim group
  const int p = pos[b];
  // Keys 0 .. p (the last window of them on sliding layers), within the cache; formed
  // without p + 1, which overflows at the largest position.
  const int kv_len = p < 0 ? 0 : min(min(p, (kSliding ? window : cap) - 1) + 1, cap);
  const int k_begin = c * chunk;
  const int k_end = min(kv_len, k_begin + chunk);

  // Q^T operand: column n16 < 4 is query head 4*kvh + n16, dims 32dc + 8g .. +7.
  const bool qlane = n16 < kGroup;
  bf16x8 qf[8];
  {
    const bf16_t* qrow = q + ((long long)b * kHq + kvh * kGroup + (qlane ? n16 : 0)) * kD + 8 * g;
#pragma unroll
    for (int dc = 0; dc < 8; ++dc)
      qf[dc] = qlane ? *reinterpret_cast<const bf16x8*>(qrow + 32 * dc) : bf16x8{};
  }
  if (rope_q && qlane) {
    // Rotate-half pairs (d, d + r/2) both live in this lane: fragment dc pairs with dc + kNdc.
#pragma unroll
    for (int dc = 0; dc < kNdc; ++dc) {
      const bf16x8 xa = qf[dc], xb = qf[dc + kNdc];
      f32x4 ya0, ya1, yb0, yb1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float sv, cv;
        sincos_angle(rope_angle(p, tab.inv_freq[32 * dc + 8 * g + e]), &sv, &cv);
        const float a = (float)xa[e], bb = (float)xb[e];
        float ya, yb;
        rope_pair(a, bb, cv, sv, &ya, &yb);
        if (e < 4) { ya0[e] = ya; yb0[e] = yb; } else { ya1[e - 4] = ya; yb1[e - 4] = yb; }
      }
      const bf16x4 a0 = __builtin_convertvector(ya0, bf16x4), a1 = __builtin_convertvector(ya1, bf16x4);
      const bf16x4 b0 = __builtin_convertvector(yb0, bf16x4), b1 = __builtin_convertvector(yb1, bf16x4);
      qf[dc] = bf16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      qf[dc + kNdc] = bf16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    }
  }

  const long long kv_off = ((long long)b * cap * kHkv + kvh) * kD;
  const bf16_t* kb = kc + kv_off;
  const bf16_t* vb = vc + kv_off;

  float m_run = -INFINITY, l_run = 0.f;
  float o[kGroup][8];
#pragma unroll
  for (int hl = 0; hl < kGroup; ++hl)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hl][e] = 0.f;

  attend_keys(qf, kb, vb, k_begin, k_end, sl2, p_lds[kvh], lane, m_run, l_run, o);

  // Fold the two key parities together, then the softmax sums over the 4 k-groups.
#pragma unroll
  for (int hl = 0; hl < kGroup; ++hl)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hl][e] += __shfl_xor(o[hl][e], 32);
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  const long long part = ((long long)(b * kHkv + kvh) * nchunks + c) * kGroup;
  if (half == 0) {
#pragma unroll
    for (int hl = 0; hl < kGroup; ++hl) {
      float* dst = ws_o + (part + hl) * kD + 8 * dg;
      *reinterpret_cast<f32x4*>(dst) = f32x4{o[hl][0], o[hl][1], o[hl][2], o[hl][3]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[hl][4], o[hl][5], o[hl][6], o[hl][7]};
    }
  }
  if (lane < kGroup) {
    ws_ml[(part + lane) * 2] = m_run;
    ws_ml[(part + lane) * 2 + 1] = l_run;
  }
}

// 8-bit KV variant of decode_split_kernel: the caches hold E4M3 codes [B, cap, 4, 256]
// with fp32 scales [B, 4, cap] per (token, KV head).  Same grid, waves and partials.
//   * QK: a lane's K fragment (8 codes of one key) is widened exactly to bf16 with the
//     hardware conversion (scale 1), the bf16 MFMA runs as before, and the key's scale
//     multiplies its score: sum_d q_d (c_d s) = s sum_d q_d c_d.
//   * PV: the value scale of key j is folded into its probability before the broadcast
//     (sum_j p_j s_j c_j); lane (kq, dg16) accumulates keys kq, kq + 4, .. of the step over
//     dims 16 dg16 .. +15, and the 4 key phases are summed at the end of the chunk.
// The softmax sum uses the unscaled probabilities.  [T5] §3.2 "Deployment steps and key
// parameters" (quantized KV cache for the 1M context).
template <bool kSliding>
__global__ __launch_bounds__(256) void decode_split_fp8_kernel(
    const bf16_t* __restrict__ q, const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
    const float* __restrict__ ksc, const float* __restrict__ vsc, int cap,
    const int* __restrict__ pos, int window, int chunk, int nchunks, float* __restrict__ ws_o,
    float* __restrict__ ws_ml, int rope_q, RopeTable tab, float sl2) {
  constexpr int kNdc = kSliding ? 4 : 1;
  __shared__ __attribute__((aligned(16))) float p_lds[kHkv][kStep][4];

  const int c = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, kvh = tid >> 6;
  const int n16 = lane & 15, g = lane >> 4;    // MFMA view: column (head) and k-group
  const int kq = lane >> 4, dg = lane & 15;    // PV view: key phase and 16-dim group
  const int p = pos[b];
  // Keys 0 .. p (the last window of them on sliding layers), within the cache; formed
  // without p + 1, which overflows at the largest position.
  const int kv_len = p < 0 ? 0 : min(min(p, (kSliding ? window : cap) - 1) + 1, cap);
  const int k_begin = c * chunk;
  const int k_end = min(kv_len, k_begin + chunk);

  const bool qlane = n16 < kGroup;
  bf16x8 qf[8];
  {
    const bf16_t* qrow = q + ((long long)b * kHq + kvh * kGroup + (qlane ? n16 : 0)) * kD + 8 * g;
#pragma unroll
    for (int dc = 0; dc < 8; ++dc)
      qf[dc] = qlane ? *reinterpret_cast<const bf16x8*>(qrow + 32 * dc) : bf16x8{};
  }
  if (rope_q && qlane) {
#pragma unroll
    for (int dc = 0; dc < kNdc; ++dc) {
      const bf16x8 xa = qf[dc], xb = qf[dc + kNdc];
      f32x4 ya0, ya1, yb0, yb1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float sv, cv;
        sincos_angle(rope_angle(p, tab.inv_freq[32 * dc + 8 * g + e]), &sv, &cv);
        float ya, yb;
        rope_pair((float)xa[e], (float)xb[e], cv, sv, &ya, &yb);
        if (e < 4) { ya0[e] = ya; yb0[e] = yb; } else { ya1[e - 4] = ya; yb1[e - 4] = yb; }
      }
      const bf16x4 a0 = __builtin_convertvector(ya0, bf16x4), a1 = __builtin_convertvector(ya1, bf16x4);
      const bf16x4 b0 = __builtin_convertvector(yb0, bf16x4), b1 = __builtin_convertvector(yb1, bf16x4);
      qf[dc] = bf16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      qf[dc + kNdc] = bf16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    }
  }

  constexpr long long rs = kHkv * kD;  // bytes per cache row (4 heads x 256 codes)
  const long long kv_off = ((long long)b * cap * kHkv + kvh) * kD;
  const uint8_t* kb = kc + kv_off;
  const uint8_t* vb = vc + kv_off;
  const float* ks = ksc + ((long long)b * kHkv + kvh) * cap;
  const float* vs = vsc + ((long long)b * kHkv + kvh) * cap;

  float m_run = -INFINITY, l_run = 0.f;
  float o[kGroup][16];
#pragma unroll
  for (int hl = 0; hl < kGroup; ++hl)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[hl][e] = 0.f;

  // Step k0's K codes, scales and V codes.  Keys past k_end read row k_end - 1 (masked
  // scores, zero probabilities), so the loads are unconditional and the compiler can count
  // them; each array is refilled for the next step as soon as this step has consumed it
  // (the last step reloads its final row), keeping loads in flight during the arithmetic.
  uint2 kraw[2][8];
  float kscale[2][4], vscale[2][4];
  uint4 vraw[8];
  auto load_k = [&](int k0) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int key = min(k0 + 16 * blk + n16, k_end - 1);
      const uint8_t* kr = kb + (long long)key * rs + 8 * g;
#pragma unroll
      for (int dc = 0; dc < 8; ++dc) kraw[blk][dc] = *reinterpret_cast<const uint2*>(kr + 32 * dc);
    }
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = min(k0 + 16 * blk + 4 * g + j, k_end - 1);
        kscale[blk][j] = ks[key];
        vscale[blk][j] = vs[key];
      }
  };
  auto load_v = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = min(k0 + kq + 4 * i, k_end - 1);
      vraw[i] = *reinterpret_cast<const uint4*>(vb + (long long)key * rs + 16 * dg);
    }
  };
  if (k_begin < k_end) {
    load_k(k_begin);
    load_v(k_begin);
  }
  for (int k0 = k_begin; k0 < k_end; k0 += kStep) {
    const int kn = min(k0 + kStep, k_end - 1);
    f32x4 sacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const uint2 w = kraw[blk][dc];
        const bf16x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false);
        const bf16x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true);
        const bf16x2 e2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false);
        const bf16x2 e3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true);
        const bf16x8 kf = bf16x8{e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
        sacc[blk] = mfma16(kf, qf[dc], sacc[blk]);
      }
    }
    float mloc = -INFINITY;
    float sv[2][4], vsc[2][4];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = k0 + 16 * blk + 4 * g + j;
        const float v = key < k_end ? sacc[blk][j] * kscale[blk][j] * sl2 : -INFINITY;
        sv[blk][j] = v;
        vsc[blk][j] = vscale[blk][j];
        mloc = fmaxf(mloc, v);
      }
    load_k(kn);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    // The reference max moves only when a step beats it by more than 2^8 (or on the first
    // visible key): probabilities stay below 256, and O is rescaled on those steps only.
    const bool bump = mloc > m_run + kRescaleLog2 || (m_run == -INFINITY && mloc != -INFINITY);
    if (__any(bump)) {
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
      // Per-head factors live in lanes 0..3 (column = head, k-group 0).
      const float a0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 0));
      const float a1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 1));
      const float a2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 2));
      const float a3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 3));
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        o[0][e] *= a0;
        o[1][e] *= a1;
        o[2][e] *= a2;
        o[3][e] *= a3;
      }
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float rsum = 0.f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pj = fast_exp2(sv[blk][j] - m_use);
        sv[blk][j] = pj;
        rsum += pj;
      }
    l_run += rsum;

    if (qlane) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          p_lds[kvh][16 * blk + 4 * g + j][n16] = sv[blk][j] * vsc[blk][j];
    }
    wave_lds_fence();
    // Keys a = kq + 8j and b = a + 4 share a lane: a byte permute interleaves their codes,
    // one conversion yields the (a, b) pair of a dim in bf16, and one dot2 adds p_a v_a +
    // p_b v_b (probabilities, with the V scales folded in, in bf16).
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 pa = *reinterpret_cast<const f32x4*>(&p_lds[kvh][kq + 8 * j][0]);
      const f32x4 pb = *reinterpret_cast<const f32x4*>(&p_lds[kvh][kq + 8 * j + 4][0]);
      bf16x2 pp[kGroup];
#pragma unroll
      for (int hl = 0; hl < kGroup; ++hl) pp[hl] = __builtin_bit_cast(bf16x2, pack_bf16x2(pa[hl], pb[hl]));
      const uint32_t va[4] = {vraw[2 * j].x, vraw[2 * j].y, vraw[2 * j].z, vraw[2 * j].w};
      const uint32_t vb2[4] = {vraw[2 * j + 1].x, vraw[2 * j + 1].y, vraw[2 * j + 1].z, vraw[2 * j + 1].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo = __builtin_amdgcn_perm(vb2[w], va[w], 0x05010400u);  // a0 b0 a1 b1
        const uint32_t hi = __builtin_amdgcn_perm(vb2[w], va[w], 0x07030602u);  // a2 b2 a3 b3
        const bf16x2 d[4] = {__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false),
                             __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true),
                             __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false),
                             __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true)};
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int hl = 0; hl < kGroup; ++hl)
            o[hl][4 * w + e] = __builtin_amdgcn_fdot2_f32_bf16(d[e], pp[hl], o[hl][4 * w + e], false);
      }
    }
    load_v(kn);
    wave_lds_fence();
  }

  // Sum the 4 key phases, then the softmax sums over the 4 k-groups.
#pragma unroll
  for (int hl = 0; hl < kGroup; ++hl)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      o[hl][e] += __shfl_xor(o[hl][e], 16);
      o[hl][e] += __shfl_xor(o[hl][e], 32);
    }
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  const long long part = ((long long)(b * kHkv + kvh) * nchunks + c) * kGroup;
  if (kq == 0) {
#pragma unroll
    for (int hl = 0; hl < kGroup; ++hl) {
      float* dst = ws_o + (part + hl) * kD + 16 * dg;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        *reinterpret_cast<f32x4*>(dst + 4 * e4) =
            f32x4{o[hl][4 * e4], o[hl][4 * e4 + 1], o[hl][4 * e4 + 2], o[hl][4 * e4 + 3]};
    }
  }
  if (lane < kGroup) {
    ws_ml[(part + lane) * 2] = m_run;
    ws_ml[(part + lane) * 2 + 1] = l_run;
  }
}

// Grid (B * 16 query heads, 256 / 32 dim slices); 256 threads = 8 four-dim quads x 32
// chunk groups, each thread loading 16 bytes of a chunk's partial output.  Pass 1: the
// largest chunk max.  Pass 2: each chunk group folds every 32nd chunk's partial with weight
// 2^(m_c - M); the 32 groups are summed through LDS.
constexpr int kCombDims = 32;
constexpr int kCombQuads = kCombDims / 4;
constexpr int kCombGroups = 256 / kCombQuads;

__global__ __launch_bounds__(256) void decode_combine_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_ml, int nchunks,
    const bf16_t* __restrict__ gate, bf16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ f32x4 red_o[kCombGroups][kCombQuads];
  __shared__ float red_l[kCombGroups];
  __shared__ float red_m[4];
  const int b = blockIdx.x / kHq, h = blockIdx.x % kHq;
  const int kvh = h / kGroup, hl = h % kGroup;
  const int dq = threadIdx.x & (kCombQuads - 1), cg = threadIdx.x / kCombQuads;
  const int d = blockIdx.y * kCombDims + 4 * dq;
  const long long base = (long long)(b * kHkv + kvh) * nchunks;

  float M = -INFINITY;
  for (int c = threadIdx.x; c < nchunks; c += 256) M = fmaxf(M, ws_ml[((base + c) * kGroup + hl) * 2]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if ((threadIdx.x & 63) == 0) red_m[threadIdx.x >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
  const float M_use = M == -INFINITY ? 0.f : M;

  // Eight chunks per batch, their loads issued before any of their arithmetic (indices
  // past the last chunk read the last one and get weight 0): the loop is bound by load
  // latency, so the chunks are spread over as many groups as the workgroup holds.
  constexpr int kBatch = 8;
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = cg; c0 < nchunks; c0 += kBatch * kCombGroups) {
    float mv[kBatch], lv[kBatch];
    f32x4 ov[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const long long pc = (base + min(c0 + u * kCombGroups, nchunks - 1)) * kGroup + hl;
      mv[u] = ws_ml[pc * 2];
      lv[u] = ws_ml[pc * 2 + 1];
      ov[u] = *reinterpret_cast<const f32x4*>(ws_o + pc * kD + d);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float wgt = c0 + u * kCombGroups < nchunks ? fast_exp2(mv[u] - M_use) : 0.f;
      L += lv[u] * wgt;
      acc += ov[u] * wgt;
    }
  }
  red_o[cg][dq] = acc;
  if (dq == 0) red_l[cg] = L;
  __syncthreads();
  if (threadIdx.x < kCombDims) {
    const int dl = threadIdx.x;
    float Lt = 0.f, at = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < kCombGroups; ++g2) {
      Lt += red_l[g2];
      at += red_o[g2][dl >> 2][dl & 3];
    }
    const long long row = (long long)b * kHq + h;
    const float g = bf16_to_f32(gate[row]);
    const float sg = 1.f / (1.f + expf(-g));
    const int dd = blockIdx.y * kCombDims + dl;
    out[row * kD + dd] = f32_to_bf16(Lt > 0.f ? at * (sg / Lt) : 0.f);
    if (dd == 0 && lse != nullptr) lse[row] = Lt > 0.f ? (M + log2f(Lt)) * kLn2 : -INFINITY;
  }
}

constexpr int kRingWaves = 4;  // waves of the fused ring step

// One decode step of a sliding layer in a single launch: append, attention over the ring
// and the merge.  Workgroup (kv head, b) rotates the new key by the token's position p and
// writes K and V to ring slot p mod 512 (the same bits as the rotating append), then
// attends query heads 4 kvh .. 4 kvh + 3 over the ring's min(p + 1, 512) filled slots: each
// of the 4 waves takes 128 slots (four of the split kernel's steps), and the 4 partials are
// merged by log-sum-exp through LDS, normalised, gated and stored as the combine does.
// The cos/sin of p * omega_i are computed once and serve both the key and the query.
// [T2] "The real bottleneck of a million-token context" (sliding layers keep the last 512
// tokens); [T3] "Sliding window 512" (RoPE theta 1e4 over all 256 dims).
// kAppend: the step's append is fused in (the schedule driver); otherwise the token's key
// and value are already in the ring (a plain sliding decode), and rope_q says whether q
// still needs its rotation.
template <bool kAppend>
__global__ __launch_bounds__(64 * kRingWaves) void ring_step_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_new,
    const bf16_t* __restrict__ v_new, bf16_t* __restrict__ k_ring, bf16_t* __restrict__ v_ring,
    const int* __restrict__ pos, const bf16_t* __restrict__ gate, bf16_t* __restrict__ out,
    float* __restrict__ lse, RopeTable tab, float sl2, int rope_q) {
  constexpr int kSlots = 512;
  constexpr int kHalf = 128;       // rot_dim / 2
  constexpr int kPerWave = kSlots / kRingWaves;
  __shared__ f32x2 cs[kHalf];
  __shared__ __attribute__((aligned(16))) float p_lds[kRingWaves][kStep][4];
  __shared__ __attribute__((aligned(16))) float part_o[kRingWaves][kGroup][kD];
  __shared__ float part_ml[kRingWaves][kGroup][2];

  const int kvh = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int half = lane >> 5, dg = lane & 31;
  const int p = pos[b];

  // The query's loads go out first; the append and its fence hide their latency.
  const bool qlane = n16 < kGroup;
  bf16x8 qf[8];
  {
    const bf16_t* qrow = q + ((long long)b * kHq + kvh * kGroup + (qlane ? n16 : 0)) * kD + 8 * g;
#pragma unroll
    for (int dc = 0; dc < 8; ++dc)
      qf[dc] = qlane ? *reinterpret_cast<const bf16x8*>(qrow + 32 * dc) : bf16x8{};
  }

  if (tid < kHalf && (kAppend || rope_q)) {
    float sv, cv;
    sincos_angle(rope_angle(p, tab.inv_freq[tid]), &sv, &cv);
    cs[tid] = f32x2{cv, sv};
  }
  __syncthreads();

  const long long ring_off = ((long long)b * kSlots * kHkv + kvh) * kD;
  if (kAppend && p >= 0) {
    const long long row = ring_off + (long long)(p & (kSlots - 1)) * kHkv * kD;
    const long long src = ((long long)b * kHkv + kvh) * kD;
    if (tid < kHalf / 8) {
      // Dims d0 .. d0 + 7 and their partners d0 + 128 .. d0 + 135.
      const int d0 = 8 * tid;
      const uint4 xa = *reinterpret_cast<const uint4*>(k_new + src + d0);
      const uint4 xb = *reinterpret_cast<const uint4*>(k_new + src + d0 + kHalf);
      const uint32_t wa[4] = {xa.x, xa.y, xa.z, xa.w};
      const uint32_t wb[4] = {xb.x, xb.y, xb.z, xb.w};
      uint32_t ya[4], yb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x2 c0 = cs[d0 + 2 * e], c1 = cs[d0 + 2 * e + 1];
        float ya0, yb0, ya1, yb1;
        rope_pair(bf16_lo(wa[e]), bf16_lo(wb[e]), c0.x, c0.y, &ya0, &yb0);
        rope_pair(bf16_hi(wa[e]), bf16_hi(wb[e]), c1.x, c1.y, &ya1, &yb1);
        ya[e] = pack_bf16x2(ya0, ya1);
        yb[e] = pack_bf16x2(yb0, yb1);
      }
      *reinterpret_cast<uint4*>(k_ring + row + d0) = uint4{ya[0], ya[1], ya[2], ya[3]};
      *reinterpret_cast<uint4*>(k_ring + row + d0 + kHalf) = uint4{yb[0], yb[1], yb[2], yb[3]};
    } else if (tid < kHalf / 8 + kD / 8) {
      const int d0 = 8 * (tid - kHalf / 8);
      *reinterpret_cast<uint4*>(v_ring + row + d0) = *reinterpret_cast<const uint4*>(v_new + src + d0);
    }
  }
  // The new row is read below by other waves of this workgroup only: the barrier's
  // workgroup-scope release and acquire make it visible (the waves share one CU), with no
  // device-scope fence, which would write back and invalidate L2.
  __syncthreads();

  // Q^T operand as in the split kernel (loaded first, above), rotated with the shared table.
  if (qlane && rope_q) {
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) {
      const bf16x8 xa = qf[dc], xb = qf[dc + 4];
      f32x4 ya0, ya1, yb0, yb1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const f32x2 c = cs[32 * dc + 8 * g + e];
        float ya, yb;
        rope_pair((float)xa[e], (float)xb[e], c.x, c.y, &ya, &yb);
        if (e < 4) { ya0[e] = ya; yb0[e] = yb; } else { ya1[e - 4] = ya; yb1[e - 4] = yb; }
      }
      const bf16x4 a0 = __builtin_convertvector(ya0, bf16x4), a1 = __builtin_convertvector(ya1, bf16x4);
      const bf16x4 b0 = __builtin_convertvector(yb0, bf16x4), b1 = __builtin_convertvector(yb1, bf16x4);
      qf[dc] = bf16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      qf[dc + 4] = bf16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    }
  }

  const int kv_len = p >= 0 ? min(p, kSlots - 1) + 1 : 0;  // no p + 1: p may be 2^31 - 1
  const int k_begin = kPerWave * w;
  const int k_end = min(kv_len, k_begin + kPerWave);
  float m_run = -INFINITY, l_run = 0.f;
  float o[kGroup][8];
#pragma unroll
  for (int hl = 0; hl < kGroup; ++hl)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hl][e] = 0.f;
  attend_keys(qf, k_ring + ring_off, v_ring + ring_off, k_begin, k_end, sl2, p_lds[w], lane,
              m_run, l_run, o);
#pragma unroll
  for (int hl = 0; hl < kGroup; ++hl)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hl][e] += __shfl_xor(o[hl][e], 32);
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (half == 0) {
#pragma unroll
    for (int hl = 0; hl < kGroup; ++hl) {
      *reinterpret_cast<f32x4*>(&part_o[w][hl][8 * dg]) = f32x4{o[hl][0], o[hl][1], o[hl][2], o[hl][3]};
      *reinterpret_cast<f32x4*>(&part_o[w][hl][8 * dg + 4]) = f32x4{o[hl][4], o[hl][5], o[hl][6], o[hl][7]};
    }
  }
  if (lane < kGroup) {
    part_ml[w][lane][0] = m_run;
    part_ml[w][lane][1] = l_run;
  }
  __syncthreads();

  // Merge: thread (head hl, dims 4j .. 4j + 3).
  const int hl = tid >> 6, d = 4 * (tid & 63);
  float M = -INFINITY;
#pragma unroll
  for (int v = 0; v < kRingWaves; ++v) M = fmaxf(M, part_ml[v][hl][0]);
  const float M_use = M == -INFINITY ? 0.f : M;
  float L = 0.f;
  f32x4 acc = f32x4{};
#pragma unroll
  for (int v = 0; v < kRingWaves; ++v) {
    const float wgt = fast_exp2(part_ml[v][hl][0] - M_use);
    L += part_ml[v][hl][1] * wgt;
    acc += *reinterpret_cast<const f32x4*>(&part_o[v][hl][d]) * wgt;
  }
  const long long row = (long long)b * kHq + kvh * kGroup + hl;
  const float gl = bf16_to_f32(gate[row]);
  const float sg = 1.f / (1.f + expf(-gl));
  const float f = L > 0.f ? sg / L : 0.f;
  *reinterpret_cast<uint2*>(out + row * kD + d) =
      uint2{pack_bf16x2(acc[0] * f, acc[1] * f), pack_bf16x2(acc[2] * f, acc[3] * f)};
  if (d == 0 && lse != nullptr) lse[row] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

constexpr int kRingSlots = 512;                     // a sliding layer's ring
constexpr int kRingSplits = 8;                      // workgroups per (KV head, sequence)
constexpr int kSplitWaves = 2;                      // waves per split workgroup
constexpr int kRingPerSplit = kRingSlots / kRingSplits;
constexpr int kRingSplitMaxB = 2;                   // larger batches use the fused kernel
static_assert(kRingPerSplit == kSplitWaves * kStep, "one 32-key step per wave");

// The same step for small batches, where one workgroup per (KV head, sequence) leaves most
// CUs idle: append, attention over the ring and the merge in one launch, with the ring's
// 512 slots split over kRingSplits workgroups per (KV head,
// sequence), so that the 512 KiB a head's ring holds stream through that many CUs: one CU
// alone reached only ~37 B/clk of it.  Every workgroup computes cos / sin of p * omega_i;
// the one whose slots hold p mod 512 rotates the new key by the token's position p and
// writes K and V to that slot (the same bits as the rotating append), and only it reads
// that slot.  Each workgroup attends query heads 4 kvh .. 4 kvh + 3 over its filled slots
// (one 32-key step per wave), merges its two waves through LDS and publishes the partial
// (reference max, sum, unnormalised o) to the workspace.  The last workgroup to arrive
// (a counter per (KV head, sequence), which it resets to zero) merges the kRingSplits
// partials by log-sum-exp, normalises, gates and stores as the combine does.
// [T2] "The real bottleneck of a million-token context" (sliding layers keep the last 512
// tokens); [T3] "Sliding window 512" (RoPE theta 1e4 over all 256 dims).
// kAppend: the step's append is fused in (the schedule driver); otherwise the token's key
// and value are already in the ring (a plain sliding decode), and rope_q says whether q
// still needs its rotation.
template <bool kAppend>
__global__ __launch_bounds__(64 * kSplitWaves) void ring_split_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_new,
    const bf16_t* __restrict__ v_new, bf16_t* __restrict__ k_ring, bf16_t* __restrict__ v_ring,
    const int* __restrict__ pos, const bf16_t* __restrict__ gate, bf16_t* __restrict__ out,
    float* __restrict__ lse, RopeTable tab, float sl2, float* __restrict__ ws_o,
    float* __restrict__ ws_ml, unsigned* __restrict__ counters, int rope_q) {
  constexpr int kHalf = 128;       // rot_dim / 2
  __shared__ f32x2 cs[kHalf];
  __shared__ __attribute__((aligned(16))) float p_lds[kSplitWaves][kStep][4];
  __shared__ __attribute__((aligned(16))) float part_o[kSplitWaves][kGroup][kD];
  __shared__ float part_ml[kSplitWaves][kGroup][2];
  __shared__ unsigned last;

  const int kvh = blockIdx.x / kRingSplits, sp = blockIdx.x % kRingSplits, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int half = lane >> 5, dg = lane & 31;
  const int p = pos[b];
  // Merge threads: head hl, dims d0 .. d0 + 7.
  const int hl = tid >> 5, d0 = 8 * (tid & 31);
  const long long row = (long long)b * kHq + kvh * kGroup + hl;
  const float gate_logit = bf16_to_f32(gate[row]);

  const bool qlane = n16 < kGroup;
  bf16x8 qf[8];
  {
    const bf16_t* qrow = q + ((long long)b * kHq + kvh * kGroup + (qlane ? n16 : 0)) * kD + 8 * g;
#pragma unroll
    for (int dc = 0; dc < 8; ++dc)
      qf[dc] = qlane ? *reinterpret_cast<const bf16x8*>(qrow + 32 * dc) : bf16x8{};
  }

  static_assert(64 * kSplitWaves >= kHalf, "one thread per frequency");
  if (tid < kHalf && (kAppend || rope_q)) {
    float sv, cv;
    sincos_angle(rope_angle(p, tab.inv_freq[tid]), &sv, &cv);
    cs[tid] = f32x2{cv, sv};
  }
  __syncthreads();

  const long long ring_off = ((long long)b * kRingSlots * kHkv + kvh) * kD;
  const int slot_new = p & (kRingSlots - 1);
  if (kAppend && p >= 0 && slot_new / kRingPerSplit == sp) {
    const long long dst = ring_off + (long long)slot_new * kHkv * kD;
    const long long src = ((long long)b * kHkv + kvh) * kD;
    if (tid < kHalf / 8) {
      // Dims d0 .. d0 + 7 and their partners d0 + 128 .. d0 + 135.
      const int d = 8 * tid;
      const uint4 xa = *reinterpret_cast<const uint4*>(k_new + src + d);
      const uint4 xb = *reinterpret_cast<const uint4*>(k_new + src + d + kHalf);
      const uint32_t wa[4] = {xa.x, xa.y, xa.z, xa.w};
      const uint32_t wb[4] = {xb.x, xb.y, xb.z, xb.w};
      uint32_t ya[4], yb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x2 c0 = cs[d + 2 * e], c1 = cs[d + 2 * e + 1];
        float ya0, yb0, ya1, yb1;
        rope_pair(bf16_lo(wa[e]), bf16_lo(wb[e]), c0.x, c0.y, &ya0, &yb0);
        rope_pair(bf16_hi(wa[e]), bf16_hi(wb[e]), c1.x, c1.y, &ya1, &yb1);
        ya[e] = pack_bf16x2(ya0, ya1);
        yb[e] = pack_bf16x2(yb0, yb1);
      }
      *reinterpret_cast<uint4*>(k_ring + dst + d) = uint4{ya[0], ya[1], ya[2], ya[3]};
      *reinterpret_cast<uint4*>(k_ring + dst + d + kHalf) = uint4{yb[0], yb[1], yb[2], yb[3]};
    } else if (tid < kHalf / 8 + kD / 8) {
      const int d = 8 * (tid - kHalf / 8);
      *reinterpret_cast<uint4*>(v_ring + dst + d) = *reinterpret_cast<const uint4*>(v_new + src + d);
    }
    // The new row is read below by this workgroup only: the barrier's workgroup-scope
    // release and acquire make it visible (its waves share one CU).
    __syncthreads();
  }

  // Q^T operand as in the split kernel (loaded first, above), rotated with the shared table.
  if (qlane && rope_q) {
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) {
      const bf16x8 xa = qf[dc], xb = qf[dc + 4];
      f32x4 ya0, ya1, yb0, yb1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const f32x2 c = cs[32 * dc + 8 * g + e];
        float ya, yb;
        rope_pair((float)xa[e], (float)xb[e], c.x, c.y, &ya, &yb);
        if (e < 4) { ya0[e] = ya; yb0[e] = yb; } else { ya1[e - 4] = ya; yb1[e - 4] = yb; }
      }
      const bf16x4 a0 = __builtin_convertvector(ya0, bf16x4), a1 = __builtin_convertvector(ya1, bf16x4);
      const bf16x4 b0 = __builtin_convertvector(yb0, bf16x4), b1 = __builtin_convertvector(yb1, bf16x4);
      qf[dc] = bf16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      qf[dc + 4] = bf16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    }
  }

  // Slots [k_begin, k_end) of this wave: the ring's first min(p + 1, 512) slots are filled
  // (formed without p + 1, which overflows at the largest position).
  const int kv_len = p >= 0 ? min(p, kRingSlots - 1) + 1 : 0;
  const int k_begin = kRingPerSplit * sp + kStep * w;
  const int k_end = min(kv_len, k_begin + kStep);
  float m_run = -INFINITY, l_run = 0.f;
  float o[kGroup][8];
#pragma unroll
  for (int h = 0; h < kGroup; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  attend_keys(qf, k_ring + ring_off, v_ring + ring_off, k_begin, k_end, sl2, p_lds[w], lane,
              m_run, l_run, o);
#pragma unroll
  for (int h = 0; h < kGroup; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] += __shfl_xor(o[h][e], 32);
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (half == 0) {
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      *reinterpret_cast<f32x4*>(&part_o[w][h][8 * dg]) = f32x4{o[h][0], o[h][1], o[h][2], o[h][3]};
      *reinterpret_cast<f32x4*>(&part_o[w][h][8 * dg + 4]) = f32x4{o[h][4], o[h][5], o[h][6], o[h][7]};
    }
  }
  if (lane < kGroup) {
    part_ml[w][lane][0] = m_run;
    part_ml[w][lane][1] = l_run;
  }
  __syncthreads();

  // This workgroup's partial: its waves merged under their largest reference max.
  const long long part = ((long long)(b * kHkv + kvh) * kRingSplits + sp) * kGroup + hl;
  {
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kSplitWaves; ++v) M = fmaxf(M, part_ml[v][hl][0]);
    const float M_use = M == -INFINITY ? 0.f : M;
    float L = 0.f;
    f32x4 a0 = f32x4{}, a1 = f32x4{};
#pragma unroll
    for (int v = 0; v < kSplitWaves; ++v) {
      const float wgt = fast_exp2(part_ml[v][hl][0] - M_use);
      L += part_ml[v][hl][1] * wgt;
      a0 += *reinterpret_cast<const f32x4*>(&part_o[v][hl][d0]) * wgt;
      a1 += *reinterpret_cast<const f32x4*>(&part_o[v][hl][d0 + 4]) * wgt;
    }
    *reinterpret_cast<f32x4*>(ws_o + part * kD + d0) = a0;
    *reinterpret_cast<f32x4*>(ws_o + part * kD + d0 + 4) = a1;
    if ((tid & 31) == 0) {
      ws_ml[2 * part] = M;
      ws_ml[2 * part + 1] = L;
    }
  }
  // Publish the partial (device-scope release), then count this workgroup in; the last one
  // of the (KV head, sequence) merges.
  __threadfence();
  __syncthreads();
  unsigned* counter = counters + b * kHkv + kvh;
  if (tid == 0) last = atomicAdd(counter, 1u) == kRingSplits - 1;
  __syncthreads();
  if (!last) return;
  __threadfence();  // acquire: every other workgroup's partial is visible

  const long long part0 = ((long long)(b * kHkv + kvh) * kRingSplits) * kGroup + hl;
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kRingSplits; ++s) M = fmaxf(M, ws_ml[2 * (part0 + s * kGroup)]);
  const float M_use = M == -INFINITY ? 0.f : M;
  float L = 0.f;
  f32x4 a0 = f32x4{}, a1 = f32x4{};
#pragma unroll
  for (int s = 0; s < kRingSplits; ++s) {
    const long long ps = part0 + s * kGroup;
    const float wgt = fast_exp2(ws_ml[2 * ps] - M_use);
    L += ws_ml[2 * ps + 1] * wgt;
    a0 += *reinterpret_cast<const f32x4*>(ws_o + ps * kD + d0) * wgt;
    a1 += *reinterpret_cast<const f32x4*>(ws_o + ps * kD + d0 + 4) * wgt;
  }
  const float sg = 1.f / (1.f + expf(-gate_logit));
  const float f = L > 0.f ? sg / L : 0.f;
  *reinterpret_cast<uint4*>(out + row * kD + d0) =
      uint4{pack_bf16x2(a0[0] * f, a0[1] * f), pack_bf16x2(a0[2] * f, a0[3] * f),
            pack_bf16x2(a1[0] * f, a1[1] * f), pack_bf16x2(a1[2] * f, a1[3] * f)};
  if ((tid & 31) == 0 && lse != nullptr) lse[row] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  if (tid == 0) *counter = 0u;  // ready for the next step (kernel boundaries order it)
}

// Clears n 32-bit counters (a kernel, not a memset, so that it can sit in a captured graph).
__global__ void zero_u32_kernel(unsigned* __restrict__ p, int n) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) p[i] = 0u;
}

}  // namespace

DecodePlan decode_plan(int B, int max_keys) {
  // One resident round: the split kernel's ~224 VGPRs leave room for two 4-wave workgroups
  // per CU, 512 on the 256-CU chip.  A second, partly filled round costs more than the
  // longer chunks do (measured at B = 1 with 2^20 keys and at B = 32 with 131073).
  constexpr int kTargetGroups = 512;
  const int steps = max(1, (max_keys + kStep - 1) / kStep);
  int nchunks = max(1, min((kTargetGroups + B - 1) / B, steps));
  const int per = (max_keys + nchunks - 1) / nchunks;
  const int chunk = max(kStep, (per + kStep - 1) / kStep * kStep);
  nchunks = max(1, (max_keys + chunk - 1) / chunk);
  return DecodePlan{nchunks, chunk};
}

hipError_t launch_decode_fp8(const bf16_t* q, const uint8_t* k_cache, const uint8_t* v_cache,
                             const float* k_scale, const float* v_scale, int cap, const int* pos,
                             int B, const bf16_t* gate, bf16_t* out, float* lse, int window,
                             bool rope_q, const RopeTable& tab, float scale_log2e,
                             const DecodePlan& plan, void* workspace, hipStream_t stream) {
  const size_t parts = (size_t)B * kHkv * plan.nchunks * kGroup;
  float* ws_o = static_cast<float*>(workspace);
  float* ws_ml = ws_o + parts * kD;
  const dim3 grid((unsigned)plan.nchunks, (unsigned)B);
  if (window > 0) {
    hipLaunchKernelGGL(decode_split_fp8_kernel<true>, grid, dim3(256), 0, stream, q, k_cache,
                       v_cache, k_scale, v_scale, cap, pos, window, plan.chunk, plan.nchunks, ws_o,
                       ws_ml, rope_q ? 1 : 0, tab, scale_log2e);
  } else {
    hipLaunchKernelGGL(decode_split_fp8_kernel<false>, grid, dim3(256), 0, stream, q, k_cache,
                       v_cache, k_scale, v_scale, cap, pos, window, plan.chunk, plan.nchunks, ws_o,
                       ws_ml, rope_q ? 1 : 0, tab, scale_log2e);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)(B * kHq), kD / kCombDims), dim3(256), 0,
                     stream, ws_o, ws_ml, plan.nchunks, gate, out, lse);
  return hipGetLastError();
}

size_t decode_workspace_bytes(int B, const DecodePlan& plan) {
  const size_t parts = (size_t)B * kHkv * plan.nchunks * kGroup;
  return parts * (kD + 2) * sizeof(float);
}

hipError_t launch_decode(const bf16_t* q, const bf16_t* k_cache, const bf16_t* v_cache, int cap,
                         const int* pos, int B, const bf16_t* gate, bf16_t* out, float* lse,
                         int window, bool rope_q, const RopeTable& tab, float scale_log2e,
                         const DecodePlan& plan, void* workspace, hipStream_t stream) {
  const size_t parts = (size_t)B * kHkv * plan.nchunks * kGroup;
  float* ws_o = static_cast<float*>(workspace);
  float* ws_ml = ws_o + parts * kD;
  const dim3 grid((unsigned)plan.nchunks, (unsigned)B);
  if (window > 0) {
    hipLaunchKernelGGL(decode_split_kernel<true>, grid, dim3(256), 0, stream, q, k_cache, v_cache,
                       cap, pos, window, plan.chunk, plan.nchunks, ws_o, ws_ml, rope_q ? 1 : 0, tab,
                       scale_log2e);
  } else {
    hipLaunchKernelGGL(decode_split_kernel<false>, grid, dim3(256), 0, stream, q, k_cache, v_cache,
                       cap, pos, window, plan.chunk, plan.nchunks, ws_o, ws_ml, rope_q ? 1 : 0, tab,
                       scale_log2e);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)(B * kHq), kD / kCombDims), dim3(256), 0,
                     stream, ws_o, ws_ml, plan.nchunks, gate, out, lse);
  return hipGetLastError();
}

size_t ring_step_workspace_bytes(int B) {
  if (B > kRingSplitMaxB) return 0;  // the fused kernel needs none
  const size_t parts = (size_t)B * kHkv * kRingSplits * kGroup;
  return parts * (kD + 2) * sizeof(float) + (size_t)B * kHkv * sizeof(unsigned);
}

hipError_t clear_ring_counters(void* workspace, int B, hipStream_t stream) {
  if (B > kRingSplitMaxB) return hipSuccess;
  const size_t parts = (size_t)B * kHkv * kRingSplits * kGroup;
  unsigned* counters = reinterpret_cast<unsigned*>(static_cast<float*>(workspace) + parts * (kD + 2));
  const int n = B * kHkv;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     counters, n);
  return hipGetLastError();
}

hipError_t launch_ring_step(const bf16_t* q, const bf16_t* k_new, const bf16_t* v_new,
                            bf16_t* k_ring, bf16_t* v_ring, const int* pos, int B,
                            const bf16_t* gate, bf16_t* out, float* lse, const RopeTable& tab,
                            float scale_log2e, void* workspace, hipStream_t stream) {
  const size_t parts = (size_t)B * kHkv * kRingSplits * kGroup;
  float* ws_o = static_cast<float*>(workspace);
  float* ws_ml = ws_o + parts * kD;
  unsigned* counters = reinterpret_cast<unsigned*>(ws_ml + parts * 2);
  // Split for B <= 2 only: each split workgroup's device-scope fence (an L2 write-back and
  // invalidate) grows with the workgroup count.  Measured per step through the driver:
  // B = 1 10.4 us split against 16.8 fused, B = 2 13.4 against 17.0, B = 4 19.6 against 17.2.
  if (B <= kRingSplitMaxB) {
    hipLaunchKernelGGL(ring_split_kernel<true>, dim3(kHkv * kRingSplits, (unsigned)B),
                       dim3(64 * kSplitWaves), 0, stream, q, k_new, v_new, k_ring, v_ring, pos,
                       gate, out, lse, tab, scale_log2e, ws_o, ws_ml, counters, 1);
  } else {
    hipLaunchKernelGGL(ring_step_kernel<true>, dim3(kHkv, (unsigned)B), dim3(64 * kRingWaves),
                       0, stream, q, k_new, v_new, k_ring, v_ring, pos, gate, out, lse, tab,
                       scale_log2e, 1);
  }
  return hipGetLastError();
}

hipError_t launch_ring_decode(const bf16_t* q, const bf16_t* k_ring, const bf16_t* v_ring,
                              const int* pos, int B, const bf16_t* gate, bf16_t* out, float* lse,
                              bool rope_q, const RopeTable& tab, float scale_log2e,
                              void* workspace, hipStream_t stream) {
  if (B > kRingSplitMaxB) {
    // The fused kernel without its append, one workgroup per (KV head, b); no workspace.
    hipLaunchKernelGGL(ring_step_kernel<false>, dim3(kHkv, (unsigned)B), dim3(64 * kRingWaves),
                       0, stream, q, nullptr, nullptr, const_cast<bf16_t*>(k_ring),
                       const_cast<bf16_t*>(v_ring), pos, gate, out, lse, tab, scale_log2e,
                       rope_q ? 1 : 0);
    return hipGetLastError();
  }
  const hipError_t e = clear_ring_counters(workspace, B, stream);
  if (e != hipSuccess) return e;
  const size_t parts = (size_t)B * kHkv * kRingSplits * kGroup;
  float* ws_o = static_cast<float*>(workspace);
  float* ws_ml = ws_o + parts * kD;
  unsigned* counters = reinterpret_cast<unsigned*>(ws_ml + parts * 2);
  // The ring is only read (k_new / v_new unused without the append).
  hipLaunchKernelGGL(ring_split_kernel<false>, dim3(kHkv * kRingSplits, (unsigned)B),
                     dim3(64 * kSplitWaves), 0, stream, q, nullptr, nullptr,
                     const_cast<bf16_t*>(k_ring), const_cast<bf16_t*>(v_ring), pos, gate, out,
                     lse, tab, scale_log2e, ws_o, ws_ml, counters, rope_q ? 1 : 0);
  return hipGetLastError();
}

bool ring_decode_applies(int B) { return B >= 1; }

}  // namespace hattn
