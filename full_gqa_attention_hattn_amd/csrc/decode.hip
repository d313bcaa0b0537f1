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
// Sliding layers instead run ring_split_kernel: one launch whose workgroups split each
// ring and whose last arriver merges their partials (with the append fused in for the
// schedule driver).  The 8-bit cache runs decode_split_fp8_kernel with the same combine.
#include "hattn_device.h"
#include "hattn_launch.h"

namespace hattn {

namespace {

constexpr int kStep = 32;  // keys per wave step
// Cache policy of a device-scope buffer access (the SC1 bit): stores are written through
// to, and loads read from, the level that all XCDs share.
constexpr int kScDevice = 16;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
constexpr float kRescaleLog2 = 8.f;  // move the reference max only when beaten by 2^8
constexpr float kLn2 = 0.69314718055994530942f;

// Lane src's value of an 8-element bf16 fragment (four 32-bit lane shuffles).
__device__ __forceinline__ bf16x8 shfl_bf16x8(bf16x8 x, int src) {
  const uint4 u = __builtin_bit_cast(uint4, x);
  return __builtin_bit_cast(bf16x8, uint4{(unsigned)__shfl((int)u.x, src), (unsigned)__shfl((int)u.y, src),
                                          (unsigned)__shfl((int)u.z, src), (unsigned)__shfl((int)u.w, src)});
}

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
// the VALU, the probabilities going through this wave's slice `pl` of LDS.  The wave
// attends NH query heads of the KV head (Q^T columns 0 .. NH - 1).
template <int NH = kGroup>
__device__ __forceinline__ void compute_step(const StepRegs& r, const bf16x8 (&qf)[8], int k0,
                                             int k_end, float sl2, float (*pl)[4], int lane,
                                             float& m_run, float& l_run, float (&o)[NH][8]) {
  static_assert(NH >= 1 && NH <= kGroup, "a wave attends at most one KV head's query heads");
  const int n16 = lane & 15, g = lane >> 4;
  const int half = lane >> 5;
  const bool qlane = n16 < NH;
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
    // Per-head factors live in lanes 0 .. NH - 1 (column = head, k-group 0).
#pragma unroll
    for (int hl = 0; hl < NH; ++hl) {
      const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), hl));
#pragma unroll
      for (int e = 0; e < 8; ++e) o[hl][e] *= a;
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
    bf16x2 pp[NH];
#pragma unroll
    for (int hl = 0; hl < NH; ++hl) pp[hl] = __builtin_bit_cast(bf16x2, pack_bf16x2(pa[hl], pb[hl]));
    const uint32_t* va = reinterpret_cast<const uint32_t*>(&r.vv[kp]);
    const uint32_t* vb2 = reinterpret_cast<const uint32_t*>(&r.vv[kp + 1]);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const bf16x2 d0 = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(vb2[w], va[w], 0x05040100u));
      const bf16x2 d1 = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(vb2[w], va[w], 0x07060302u));
#pragma unroll
      for (int hl = 0; hl < NH; ++hl) {
        o[hl][2 * w] = __builtin_amdgcn_fdot2_f32_bf16(d0, pp[hl], o[hl][2 * w], false);
        o[hl][2 * w + 1] = __builtin_amdgcn_fdot2_f32_bf16(d1, pp[hl], o[hl][2 * w + 1], false);
      }
    }
  }
  wave_lds_fence();
}

// One wave's pass over keys [k_begin, k_end) of its KV head, one 32-key step at a time.
// Leaves this lane's share of the partial (reference max, sum, o[head][8 dims]) of the NH
// query heads it attends.
template <int NH = kGroup>
__device__ __forceinline__ void attend_keys(const bf16x8 (&qf)[8], const bf16_t* kb,
                                            const bf16_t* vb, int k_begin, int k_end, float sl2,
                                            float (*pl)[4], int lane, float& m_run, float& l_run,
                                            float (&o)[NH][8]) {
  for (int k0 = k_begin; k0 < k_end; k0 += kStep) {
    StepRegs r;
    load_step(r, kb, vb, k0, k_end, lane);
    compute_step<NH>(r, qf, k0, k_end, sl2, pl, lane, m_run, l_run, o);
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
    for (int dc = 0; dc < kNdc; ++dc)
      rope_fragments(qf[dc], qf[dc + kNdc], [&](int e) {
        float sv, cv;
        sincos_angle(rope_angle(p, tab.inv_freq[32 * dc + 8 * g + e]), &sv, &cv);
        return f32x2{cv, sv};
      });
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
//   * PV on MFMA too: O^T += V^T P^T on v_mfma_f32_16x16x32_bf16, one MFMA per 16 dims.
//     The value scale of key j is folded into its probability before the broadcast
//     (sum_j p_j s_j c_j).  Lane (kq = lane / 16, i = lane mod 16) holds the 16 codes of
//     dims 16 i .. 16 i + 15 of keys kq, kq + 4, .., kq + 28 of the step: that is the V^T
//     operand of 16 MFMAs, MFMA e covering dims 16 i + e with K-index 8 kq + m being key
//     kq + 4m.  The codes are widened exactly to bf16 two at a time and one byte permute
//     pairs a dim of two keys.  The probabilities reach the P^T operand through LDS in that
//     key order.  This replaced VALU dot products (v_dot2_f32_bf16, 352 VALU operations per
//     32-key step), which left the kernel bound by VALU issue: 397 -> 377 us at 2^20 keys.
// The softmax sum uses the unscaled probabilities.  [T5] §3.2 "Deployment steps and key
// parameters" (quantized KV cache for the 1M context).
template <bool kSliding>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_split_fp8_kernel(
    const bf16_t* __restrict__ q, const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
    const float* __restrict__ ksc, const float* __restrict__ vsc, int cap,
    const int* __restrict__ pos, int window, int chunk, int nchunks, float* __restrict__ ws_o,
    float* __restrict__ ws_ml, int rope_q, RopeTable tab, float sl2) {
  constexpr int kNdc = kSliding ? 4 : 1;
  // Per wave: probability of step key j for head h at [h][8 (j mod 4) + j / 4].
  __shared__ __attribute__((aligned(16))) float p_lds[kHkv][kGroup][kStep];

  const int c = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, kvh = tid >> 6;
  const int n16 = lane & 15, g = lane >> 4;    // MFMA view: column (head) and k-group
  const int kq = lane >> 4;                    // V load view: key phase and 16-dim group
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
    for (int dc = 0; dc < kNdc; ++dc)
      rope_fragments(qf[dc], qf[dc + kNdc], [&](int e) {
        float sv, cv;
        sincos_angle(rope_angle(p, tab.inv_freq[32 * dc + 8 * g + e]), &sv, &cv);
        return f32x2{cv, sv};
      });
  }

  // K loads take 16 contiguous codes a lane: MFMA dc covers, in lane group g, dims
  // 64 (dc >> 1) + 16 g + 8 (dc & 1) .. + 7, so MFMAs 2m and 2m + 1 read one 16-byte piece.
  // Q^T moves to the same mapping once (it was loaded and rotated as dims 32 dc + 8 g, where
  // each rotary pair sits in one lane): new (g, dc) is old fragment 2 (dc >> 1) + (g >> 1)
  // of lane group 2 (g & 1) + (dc & 1), same column.
  {
    bf16x8 qn[8];
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) {
      const int src = n16 + 16 * (2 * (g & 1) + (dc & 1));
      const bf16x8 v0 = shfl_bf16x8(qf[2 * (dc >> 1)], src);
      const bf16x8 v1 = shfl_bf16x8(qf[2 * (dc >> 1) + 1], src);
      qn[dc] = (g >> 1) ? v1 : v0;
    }
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) qf[dc] = qn[dc];
  }

  constexpr long long rs = kHkv * kD;  // bytes per cache row (4 heads x 256 codes)
  const long long kv_off = ((long long)b * cap * kHkv + kvh) * kD;
  const uint8_t* kb = kc + kv_off;
  const uint8_t* vb = vc + kv_off;
  const float* ks = ksc + ((long long)b * kHkv + kvh) * cap;
  const float* vs = vsc + ((long long)b * kHkv + kvh) * cap;

  float m_run = -INFINITY, l_run = 0.f;
  // O^T accumulators: oacc[e][jj] of lane (column n16 = head, g) is dim 16 (4 g + jj) + e.
  f32x4 oacc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) oacc[e] = f32x4{};

  // Step k0's K codes, scales and V codes.  Keys past k_end read row k_end - 1 (masked
  // scores, zero probabilities), so the loads are unconditional and the compiler can count
  // them; each array is refilled for the next step as soon as this step has consumed it
  // (the last step reloads its final row), keeping loads in flight during the arithmetic.
  uint4 kraw[2][4];
  f32x4 kscale[2], vscale[2];
  // Scales of keys k0 + 16 blk + 4 g .. + 3 (consecutive in the [B, 4, cap] arrays) as one
  // 16-byte buffer load when cap keeps them 16-byte aligned; the buffer's range ends at the
  // row's cap keys (reads past it return zero).  Keys past k_end are masked below.
  // (Byte offsets and the range are 32-bit: capacities from 2^29 keys take the per-key path.)
  const bool vec_scales = (cap & 3) == 0 && cap < (1 << 29);
  const int scale_bytes = vec_scales ? cap * 4 : 0;
  const __amdgpu_buffer_rsrc_t ks_rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(ks), (short)0, scale_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vs_rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(vs), (short)0, scale_bytes, 0x00020000);
  uint4 vraw[8];
  auto load_k = [&](int k0) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int key = min(k0 + 16 * blk + n16, k_end - 1);
      const uint8_t* kr = kb + (long long)key * rs + 16 * g;
#pragma unroll
      for (int m = 0; m < 4; ++m) kraw[blk][m] = *reinterpret_cast<const uint4*>(kr + 64 * m);
    }
    if (vec_scales) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int off = 4 * (k0 + 16 * blk + 4 * g);
        kscale[blk] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ks_rs, off, 0, 0));
        vscale[blk] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(vs_rs, off, 0, 0));
      }
    } else {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = min(k0 + 16 * blk + 4 * g + j, k_end - 1);
          kscale[blk][j] = ks[key];
          vscale[blk][j] = vs[key];
        }
    }
  };
  auto load_v = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = min(k0 + kq + 4 * i, k_end - 1);
      vraw[i] = *reinterpret_cast<const uint4*>(vb + (long long)key * rs + 16 * n16);
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
        const uint4 w4 = kraw[blk][dc >> 1];
        const uint32_t wx = (dc & 1) ? w4.z : w4.x, wy = (dc & 1) ? w4.w : w4.y;
        const bf16x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wx, 1.0f, false);
        const bf16x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wx, 1.0f, true);
        const bf16x2 e2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wy, 1.0f, false);
        const bf16x2 e3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wy, 1.0f, true);
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
        // masked keys may read scales of rows never written: zero, so no NaN meets P = 0
        vsc[blk][j] = key < k_end ? vscale[blk][j] : 0.f;
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
      // Each lane's accumulators belong to its own column (head), whose factor it holds.
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[e] *= alpha;
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
          p_lds[kvh][n16][8 * j + 4 * blk + g] = sv[blk][j] * vsc[blk][j];
    }
    wave_lds_fence();
    // P^T operand: lane (column n16, k-group g) takes K-indices 8g .. 8g + 7, i.e. keys g,
    // g + 4, .., g + 28, at slots 8g .. 8g + 7 (columns past the 4 heads read a head's
    // row; those output columns are never stored).
    bf16x8 pf;
    {
      const float* prow = &p_lds[kvh][n16 & (kGroup - 1)][8 * g];
      const f32x4 pa = *reinterpret_cast<const f32x4*>(prow);
      const f32x4 pb = *reinterpret_cast<const f32x4*>(prow + 4);
      const bf16x4 lo = __builtin_convertvector(pa, bf16x4), hi = __builtin_convertvector(pb, bf16x4);
      pf = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    // V^T operand of MFMA e = 4w + 2hf + bs: element m (K-index 8 kq + m) is dim 16 dg + e
    // of key kq + 4m, code byte e of vraw[m].  Each code word is widened to two bf16 pairs
    // (dims 4w, 4w + 1 and 4w + 2, 4w + 3 of one key); a permute then pairs one dim of keys
    // 2t and 2t + 1.
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t x[8][2];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const uint32_t d = w == 0 ? vraw[m].x : w == 1 ? vraw[m].y : w == 2 ? vraw[m].z : vraw[m].w;
        x[m][0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.0f, false));
        x[m][1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.0f, true));
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int bs = 0; bs < 2; ++bs) {
          const uint32_t sel = bs ? 0x07060302u : 0x05040100u;  // high or low bf16 of each
          const uint32_t a0 = __builtin_amdgcn_perm(x[1][hf], x[0][hf], sel);
          const uint32_t a1 = __builtin_amdgcn_perm(x[3][hf], x[2][hf], sel);
          const uint32_t a2 = __builtin_amdgcn_perm(x[5][hf], x[4][hf], sel);
          const uint32_t a3 = __builtin_amdgcn_perm(x[7][hf], x[6][hf], sel);
          const int e = 4 * w + 2 * hf + bs;
          oacc[e] = mfma16(__builtin_bit_cast(bf16x8, uint4{a0, a1, a2, a3}), pf, oacc[e]);
        }
    }
    load_v(kn);
    wave_lds_fence();
  }

  // The softmax sums over the 4 k-groups.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  const long long part = ((long long)(b * kHkv + kvh) * nchunks + c) * kGroup;
  if (qlane) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float* dst = ws_o + (part + n16) * kD + 16 * (4 * g + jj);
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        *reinterpret_cast<f32x4*>(dst + 4 * e4) =
            f32x4{oacc[4 * e4][jj], oacc[4 * e4 + 1][jj], oacc[4 * e4 + 2][jj], oacc[4 * e4 + 3][jj]};
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

constexpr int kRingSlots = 512;  // a sliding layer's ring

// Workgroups per (sequence, KV head) of the ring kernel for B sequences.  Measured per
// call inside a captured graph, cold rings: 8 splits of 2 waves are fastest up to B = 8
// (10.1 us at B = 1, 11.6 at 8), 4 of 4 waves above (13.6 us at 16, 19.9 at 32, where
// 8 splits took 22.5).  One workgroup per (sequence, KV head), or one per pair of query
// heads reading the whole ring, took 17.0 us at B = 1 and 21.4 at 32: a CU alone
// streams only ~37 B/clk, so a head's 512 KiB ring has to spread over several.
int ring_splits(int B) { return B <= 8 ? 8 : 4; }

// Attention over a sliding layer's ring in one launch, for any batch: the 512 slots of
// each (sequence, KV head) are split over kRingSplits workgroups of kSplitWaves waves, one
// 32-slot step per wave.  Each wave issues its slots' loads first, before the position
// is known (every slot is addressable; unfilled ones are masked afterwards, their values
// zeroed so that NaN contents never reach the sum).  Every workgroup computes cos / sin
// of p * omega_i; with kAppend, the one whose slots hold p mod 512 rotates the new key by
// p and writes K and V to that slot (the same bits as the rotating append), and the lanes
// holding that slot take it from LDS.  Each workgroup attends query heads 4 kvh ..
// 4 kvh + 3, merges its waves through LDS and publishes the partial (reference max, sum,
// unnormalised o) to the workspace with device-scope stores.  The last workgroup to
// arrive (a counter per (sequence, KV head), which it resets to zero) merges the
// kRingSplits partials by log-sum-exp, normalises, gates and stores as the combine does.
// [T2] "The real bottleneck of a million-token context" (sliding layers keep the last 512
// tokens); [T3] "Sliding window 512" (RoPE theta 1e4 over all 256 dims).
// kAppend: the step's append is fused in (the schedule driver); otherwise the token's key
// and value are already in the ring (a plain sliding decode), and rope_q says whether q
// still needs its rotation.
template <bool kAppend, int kRingSplits, int kSplitWaves>
__global__ __launch_bounds__(64 * kSplitWaves) void ring_split_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_new,
    const bf16_t* __restrict__ v_new, bf16_t* __restrict__ k_ring, bf16_t* __restrict__ v_ring,
    const int* __restrict__ pos, const bf16_t* __restrict__ gate, bf16_t* __restrict__ out,
    float* __restrict__ lse, RopeTable tab, float sl2, float* __restrict__ ws_o,
    float* __restrict__ ws_ml, unsigned* __restrict__ counters, int rope_q) {
  constexpr int kHalf = 128;       // rot_dim / 2
  constexpr int kRingPerSplit = kRingSlots / kRingSplits;
  static_assert(kRingPerSplit == kSplitWaves * kStep, "one 32-key step per wave");
  static_assert(64 * kSplitWaves >= kHalf / 8 + kD / 8, "append threads");
  __shared__ f32x2 cs[kHalf];
  __shared__ __attribute__((aligned(16))) float p_lds[kSplitWaves][kStep][4];
  __shared__ __attribute__((aligned(16))) float part_o[kSplitWaves][kGroup][kD];
  __shared__ float part_ml[kSplitWaves][kGroup][2];
  __shared__ uint4 new_k[kD / 8], new_v[kD / 8];   // the appended row, 8 dims per entry
  __shared__ unsigned last;

  const int kvh = blockIdx.x / kRingSplits, sp = blockIdx.x % kRingSplits, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int half = lane >> 5, dg = lane & 31;
  const int p = pos[b];
  // Merge threads (the first 32 kGroup): head hl, dims d0 .. d0 + 7.
  static_assert(64 * kSplitWaves >= 32 * kGroup, "a merge thread per 8 dims of each head");
  const bool mt = tid < 32 * kGroup;
  const int hl = (tid >> 5) & (kGroup - 1), d0 = 8 * (tid & 31);
  const long long row = (long long)b * kHq + kvh * kGroup + hl;
  const float gate_logit = bf16_to_f32(gate[row]);
  // Read before the ring's loads go out (a dynamically indexed kernel argument is a memory
  // load, and waiting for it must not wait for them).
  static_assert(64 * kSplitWaves >= kHalf, "one thread per frequency");
  const float inv_freq = tab.inv_freq[tid & (kHalf - 1)];

  // Q^T operand: lanes n16 >= 4 load head 0 again (unconditional loads, so that no
  // branch around a load makes the wave wait for it); their S^T columns repeat head 0's
  // and nothing reads them.
  const bool qlane = n16 < kGroup;
  bf16x8 qf[8];
  {
    const bf16_t* qrow = q + ((long long)b * kHq + kvh * kGroup + (qlane ? n16 : 0)) * kD + 8 * g;
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) qf[dc] = *reinterpret_cast<const bf16x8*>(qrow + 32 * dc);
  }
  // The token's key (threads 0 .. 15: dims 8t .. 8t + 7 and their partners 8t + 128 ..)
  // and value (threads 16 .. 47: dims 8 (t - 16) ..), loaded whichever workgroup appends.
  const long long src = ((long long)b * kHkv + kvh) * kD;
  uint4 xa = uint4{}, xb = uint4{};
  if (kAppend) {
    // Unconditional too: every thread reads an in-range entry, threads 48 .. drop theirs.
    const int t = tid & 63;
    const bf16_t* ks = k_new + src + 8 * (t & (kHalf / 8 - 1));
    const bf16_t* vs = v_new + src + 8 * ((t - kHalf / 8) & (kD / 8 - 1));
    const uint4 ka = *reinterpret_cast<const uint4*>(ks);
    const uint4 kb2 = *reinterpret_cast<const uint4*>(ks + kHalf);
    const uint4 va = *reinterpret_cast<const uint4*>(vs);
    xa = t < kHalf / 8 ? ka : va;
    xb = kb2;
  }
  // This wave's 32 slots go out next, before the position is known: every slot of the
  // ring is addressable, and what the position rules out is masked once it is known.  The
  // loads above stay ahead of them (the memory counter is waited on in issue order).
  __builtin_amdgcn_sched_barrier(0);
  const long long ring_off = ((long long)b * kRingSlots * kHkv + kvh) * kD;
  const int k_begin = kRingPerSplit * sp + kStep * w;
  StepRegs r;
  load_step(r, k_ring + ring_off, v_ring + ring_off, k_begin, k_begin + kStep, lane);
  __builtin_amdgcn_sched_barrier(0);

  {
    // Every thread evaluates it (no branch for the frequency's load to sink into).
    float sv, cv;
    sincos_angle(rope_angle(p, inv_freq), &sv, &cv);
    if (tid < kHalf && (kAppend || rope_q)) cs[tid] = f32x2{cv, sv};
  }
  __syncthreads();

  const int slot_new = p & (kRingSlots - 1);
  const bool appends = kAppend && p >= 0 && slot_new / kRingPerSplit == sp;
  if (appends) {
    // Rotate the key by p and write K and V to slot p mod 512 (the same bits as the
    // rotating append), and keep the row in LDS for the lanes that hold that slot.
    const long long dst = ring_off + (long long)slot_new * kHkv * kD;
    if (tid < kHalf / 8) {
      const int d = 8 * tid;
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
      const uint4 ka = uint4{ya[0], ya[1], ya[2], ya[3]}, kb2 = uint4{yb[0], yb[1], yb[2], yb[3]};
      *reinterpret_cast<uint4*>(k_ring + dst + d) = ka;
      *reinterpret_cast<uint4*>(k_ring + dst + d + kHalf) = kb2;
      new_k[tid] = ka;
      new_k[tid + kHalf / 8] = kb2;
    } else if (tid < kHalf / 8 + kD / 8) {
      const int e = tid - kHalf / 8;
      *reinterpret_cast<uint4*>(v_ring + dst + 8 * e) = xa;
      new_v[e] = xa;
    }
    __syncthreads();
  }

  // Q^T rotated with the shared table (every lane, so that the repeats stay head 0's).
  if (rope_q) {
#pragma unroll
    for (int dc = 0; dc < 4; ++dc)
      rope_fragments(qf[dc], qf[dc + 4], [&](int e) { return cs[32 * dc + 8 * g + e]; });
  }

  // Slots [k_begin, k_end) of this wave: the ring's first min(p + 1, 512) slots are filled
  // (formed without p + 1, which overflows at the largest position).
  const int kv_len = p >= 0 ? min(p, kRingSlots - 1) + 1 : 0;
  const int k_end = min(kv_len, k_begin + kStep);
  if (k_end < k_begin + kStep) {
    // Unfilled slots may hold anything (NaN included): their scores are masked to -inf,
    // and their values are zeroed so that a zero probability meets a zero.
#pragma unroll
    for (int kp = 0; kp < 16; ++kp)
      if (k_begin + 2 * kp + half >= k_end) r.vv[kp] = uint4{0u, 0u, 0u, 0u};
  }
  if (appends && (unsigned)(slot_new - k_begin) < (unsigned)kStep) {
    // The lanes holding the new slot take it from LDS (their loads went out before it
    // was written).  MFMA view: lane (n16, g) holds dims 8g + 32dc .. of key
    // k_begin + 16 blk + n16; PV view: lane (half, dg) holds dims 8dg .. of key
    // k_begin + 2kp + half.
    const int j = slot_new - k_begin;
    if (n16 == (j & 15)) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
        if (blk == (j >> 4)) {
#pragma unroll
          for (int dc = 0; dc < 8; ++dc) r.kf[blk][dc] = __builtin_bit_cast(bf16x8, new_k[g + 4 * dc]);
        }
    }
    if (half == (j & 1)) {
#pragma unroll
      for (int kp = 0; kp < 16; ++kp)
        if (kp == (j >> 1)) r.vv[kp] = new_v[dg];
    }
  }
  float m_run = -INFINITY, l_run = 0.f;
  float o[kGroup][8];
#pragma unroll
  for (int h = 0; h < kGroup; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  if (k_end > k_begin)
    compute_step(r, qf, k_begin, k_end, sl2, p_lds[w], lane, m_run, l_run, o);
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

  // The partials of this (sequence, KV head): kRingSplits x 4 heads x (256 o + 2) floats,
  // addressed from their own base so every buffer offset stays small.
  const long long group = (long long)(b * kHkv + kvh) * kRingSplits * kGroup;
  const __amdgpu_buffer_rsrc_t o_rs =
      __builtin_amdgcn_make_buffer_rsrc(ws_o + group * kD, (short)0, 0x7fffffff, 0x00020000);
  const __amdgpu_buffer_rsrc_t ml_rs =
      __builtin_amdgcn_make_buffer_rsrc(ws_ml + group * 2, (short)0, 0x7fffffff, 0x00020000);
  const int o_off = ((sp * kGroup + hl) * kD + d0) * 4;   // bytes
  const int ml_off = (sp * kGroup + hl) * 8;
  // This workgroup's partial: its waves merged under their largest reference max.
  if (mt) {
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
    // Device-scope stores (sc1): written through to the level every XCD's accesses
    // meet, and acknowledged only once they are there.
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, a0), o_rs, o_off, 0, kScDevice);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, a1), o_rs, o_off + 16, 0,
                                           kScDevice);
    if ((tid & 31) == 0)
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(M), __float_as_uint(L)}, ml_rs,
                                            ml_off, 0, kScDevice);
  }
  // Every thread's partial stores are complete before the workgroup counts itself in, so
  // the last to arrive finds all of them at the device level; no L2 write-back or
  // invalidate is needed (a device-scope __threadfence would write back and invalidate
  // the whole L2 of this XCD, once per workgroup).
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  unsigned* counter = counters + b * kHkv + kvh;
  if (tid == 0)
    last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           kRingSplits - 1;
  __syncthreads();
  if (!last || !mt) return;

  // Device-scope loads (sc1) of the other workgroups' partials: never served from a line
  // cached before they were written.
  float mv[kRingSplits], lv[kRingSplits];
#pragma unroll
  for (int s = 0; s < kRingSplits; ++s) {
    const u32x2 ml =
        __builtin_amdgcn_raw_buffer_load_b64(ml_rs, (s * kGroup + hl) * 8, 0, kScDevice);
    mv[s] = __uint_as_float(ml[0]);
    lv[s] = __uint_as_float(ml[1]);
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kRingSplits; ++s) M = fmaxf(M, mv[s]);
  const float M_use = M == -INFINITY ? 0.f : M;
  float L = 0.f;
  f32x4 a0 = f32x4{}, a1 = f32x4{};
#pragma unroll
  for (int s = 0; s < kRingSplits; ++s) {
    const int off = ((s * kGroup + hl) * kD + d0) * 4;
    const f32x4 o0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(o_rs, off, 0, kScDevice));
    const f32x4 o1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(o_rs, off + 16, 0, kScDevice));
    const float wgt = fast_exp2(mv[s] - M_use);
    L += lv[s] * wgt;
    a0 += o0 * wgt;
    a1 += o1 * wgt;
  }
  const float sg = 1.f / (1.f + expf(-gate_logit));
  const float f = L > 0.f ? sg / L : 0.f;
  *reinterpret_cast<uint4*>(out + row * kD + d0) =
      uint4{pack_bf16x2(a0[0] * f, a0[1] * f), pack_bf16x2(a0[2] * f, a0[3] * f),
            pack_bf16x2(a1[0] * f, a1[1] * f), pack_bf16x2(a1[2] * f, a1[3] * f)};
  if ((tid & 31) == 0 && lse != nullptr) lse[row] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  if (tid == 0)  // ready for the next step (kernel boundaries order it)
    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  // Full layers only: a sliding layer decodes through the ring kernels (launch_ring_decode).
  if (window > 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(decode_split_kernel<false>, grid, dim3(256), 0, stream, q, k_cache, v_cache,
                     cap, pos, window, plan.chunk, plan.nchunks, ws_o, ws_ml, rope_q ? 1 : 0, tab,
                     scale_log2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)(B * kHq), kD / kCombDims), dim3(256), 0,
                     stream, ws_o, ws_ml, plan.nchunks, gate, out, lse);
  return hipGetLastError();
}

size_t ring_step_workspace_bytes(int B) {
  const size_t parts = (size_t)B * kHkv * ring_splits(B) * kGroup;
  return parts * (kD + 2) * sizeof(float) + (size_t)B * kHkv * sizeof(unsigned);
}

namespace {

// The ring kernel's partials and counters in a workspace of ring_step_workspace_bytes(B).
struct RingWs {
  float* o;
  float* ml;
  unsigned* counters;
};
RingWs ring_ws(void* workspace, int B) {
  const size_t parts = (size_t)B * kHkv * ring_splits(B) * kGroup;
  float* o = static_cast<float*>(workspace);
  return RingWs{o, o + parts * kD, reinterpret_cast<unsigned*>(o + parts * (kD + 2))};
}

template <bool kAppend>
hipError_t launch_ring_split(const bf16_t* q, const bf16_t* k_new, const bf16_t* v_new,
                             bf16_t* k_ring, bf16_t* v_ring, const int* pos, int B,
                             const bf16_t* gate, bf16_t* out, float* lse, const RopeTable& tab,
                             float scale_log2e, void* workspace, int rope_q, hipStream_t stream) {
  const RingWs ws = ring_ws(workspace, B);
  // splits x waves = 16: one 32-key step per wave over the 512 slots.
  if (ring_splits(B) == 8) {
    hipLaunchKernelGGL((ring_split_kernel<kAppend, 8, 2>), dim3(kHkv * 8, (unsigned)B),
                       dim3(64 * 2), 0, stream, q, k_new, v_new, k_ring, v_ring, pos, gate, out,
                       lse, tab, scale_log2e, ws.o, ws.ml, ws.counters, rope_q);
  } else {
    hipLaunchKernelGGL((ring_split_kernel<kAppend, 4, 4>), dim3(kHkv * 4, (unsigned)B),
                       dim3(64 * 4), 0, stream, q, k_new, v_new, k_ring, v_ring, pos, gate, out,
                       lse, tab, scale_log2e, ws.o, ws.ml, ws.counters, rope_q);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t clear_ring_counters(void* workspace, int B, hipStream_t stream) {
  unsigned* counters = ring_ws(workspace, B).counters;
  const int n = B * kHkv;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     counters, n);
  return hipGetLastError();
}

hipError_t launch_ring_step(const bf16_t* q, const bf16_t* k_new, const bf16_t* v_new,
                            bf16_t* k_ring, bf16_t* v_ring, const int* pos, int B,
                            const bf16_t* gate, bf16_t* out, float* lse, const RopeTable& tab,
                            float scale_log2e, void* workspace, hipStream_t stream) {
  return launch_ring_split<true>(q, k_new, v_new, k_ring, v_ring, pos, B, gate, out, lse, tab,
                                 scale_log2e, workspace, 1, stream);
}

hipError_t launch_ring_decode(const bf16_t* q, const bf16_t* k_ring, const bf16_t* v_ring,
                              const int* pos, int B, const bf16_t* gate, bf16_t* out, float* lse,
                              bool rope_q, const RopeTable& tab, float scale_log2e,
                              void* workspace, hipStream_t stream) {
  const hipError_t e = clear_ring_counters(workspace, B, stream);
  if (e != hipSuccess) return e;
  // The ring is only read (k_new / v_new unused without the append).
  return launch_ring_split<false>(q, nullptr, nullptr, const_cast<bf16_t*>(k_ring),
                                  const_cast<bf16_t*>(v_ring), pos, B, gate, out, lse, tab,
                                  scale_log2e, workspace, rope_q ? 1 : 0, stream);
}

}  // namespace hattn
