// RoPE (in place on Q and/or K) and the KV-cache append for one hybrid-attention layer.
//
// RoPE: [T1] "Per-layer RoPE and the local/global split" -- each layer type has its own
// rope_theta and partial_rotary_factor, cos/sin are computed per layer type from the
// token positions; [T3] "Global attention + 5M-base RoPE" -- full layers rotate only the
// first 64 of 256 dims.  Pairing is rotate-half: (i, i + r/2) for i < r/2.
//
// Append: [T2] "The real bottleneck of a million-token context" -- sliding layers keep
// only the latest 512 tokens' keys and values (a ring indexed by position mod 512), full
// layers keep every token (slot = position).
#include "hattn_device.h"
#include "hattn_launch.h"

namespace hattn {

namespace {

constexpr int kRopeTokens = 4;   // tokens per workgroup
constexpr int kRopeThreads = 256;

// One workgroup rotates kRopeTokens consecutive tokens (flattened b*S + s).  The cos/sin
// of each (token, frequency) is computed once into LDS and shared by the 16 query heads
// and 4 key heads.  Each work item turns 8 pairs: 16 bytes at d and 16 bytes at d + r/2.
// Work items cover only the heads present (K alone when q is null, and so on).

// Row and first dim of work item e; null when its token is past the end.
__device__ __forceinline__ bf16_t* rope_item(bf16_t* q, bf16_t* k, long long tok0,
                                             long long ntok, int e, int h_lo, int groups,
                                             int per_tok, int* t_out, int* d0_out) {
  const int t = e / per_tok;
  const int rem = e - t * per_tok;
  const int hh = h_lo + rem / groups, gi = rem - (hh - h_lo) * groups;
  const long long tok = tok0 + t;
  *t_out = t;
  *d0_out = gi * 8;
  if (tok >= ntok) return nullptr;
  return hh < kHq ? q + (tok * kHq + hh) * kD : k + (tok * kHkv + (hh - kHq)) * kD;
}

__global__ __launch_bounds__(kRopeThreads) void rope_qk_kernel(
    bf16_t* __restrict__ q, bf16_t* __restrict__ k, const int* __restrict__ pos0, int S,
    long long ntok, RopeTable tab) {
  __shared__ f32x2 cs[kRopeTokens][kMaxHalfRot];
  const int half = tab.rot_dim >> 1;
  const long long tok0 = (long long)blockIdx.x * kRopeTokens;
  // Read first: loads complete in issue order, so a later frequency load would also wait
  // for the rows below.  With kRopeThreads a multiple of r/2 a thread's table column is
  // the same on every pass.
  const bool one_col = kRopeThreads % half == 0;
  const float freq0 = tab.inv_freq[threadIdx.x % half];

  const int h_lo = q == nullptr ? kHq : 0;
  const int h_hi = k == nullptr ? kHq : kHq + kHkv;
  const int groups = half >> 3;                 // 8 pairs per item
  const int per_tok = (h_hi - h_lo) * groups;
  const int items = kRopeTokens * per_tok;

  // The first item's rows are loaded before the table, so their latency overlaps it.
  int t1 = 0, d1 = 0;
  bf16_t* row1 = (int)threadIdx.x < items
                     ? rope_item(q, k, tok0, ntok, threadIdx.x, h_lo, groups, per_tok, &t1, &d1)
                     : nullptr;
  uint4 xa1{}, xb1{};
  if (row1 != nullptr) {
    xa1 = *reinterpret_cast<const uint4*>(row1 + d1);
    xb1 = *reinterpret_cast<const uint4*>(row1 + d1 + half);
  }

  for (int e = threadIdx.x; e < kRopeTokens * half; e += kRopeThreads) {
    const int t = e / half, f = e - t * half;
    const long long tok = tok0 + t;
    if (tok < ntok) {
      const int b = (int)(tok / S), s = (int)(tok - (long long)b * S);
      const int p = pos0[b] + s;
      float sv, cv;
      sincos_angle(rope_angle(p, one_col ? freq0 : tab.inv_freq[f]), &sv, &cv);
      cs[t][f] = f32x2{cv, sv};
    }
  }
  __syncthreads();

  for (int e = threadIdx.x; e < items; e += kRopeThreads) {
    int t, d0;
    bf16_t* row;
    uint4 xa, xb;
    if (e == (int)threadIdx.x) {
      row = row1; t = t1; d0 = d1; xa = xa1; xb = xb1;
    } else {
      row = rope_item(q, k, tok0, ntok, e, h_lo, groups, per_tok, &t, &d0);
      if (row != nullptr) {
        xa = *reinterpret_cast<const uint4*>(row + d0);
        xb = *reinterpret_cast<const uint4*>(row + d0 + half);
      }
    }
    if (row == nullptr) continue;
    uint32_t wa[4] = {xa.x, xa.y, xa.z, xa.w};
    uint32_t wb[4] = {xb.x, xb.y, xb.z, xb.w};
    uint32_t ya[4], yb[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f32x2 c0 = cs[t][d0 + 2 * w], c1 = cs[t][d0 + 2 * w + 1];
      const float a0 = bf16_lo(wa[w]), a1 = bf16_hi(wa[w]);
      const float b0 = bf16_lo(wb[w]), b1 = bf16_hi(wb[w]);
      float ya0, yb0, ya1, yb1;
      rope_pair(a0, b0, c0.x, c0.y, &ya0, &yb0);
      rope_pair(a1, b1, c1.x, c1.y, &ya1, &yb1);
      ya[w] = pack_bf16x2(ya0, ya1);
      yb[w] = pack_bf16x2(yb0, yb1);
    }
    *reinterpret_cast<uint4*>(row + d0) = uint4{ya[0], ya[1], ya[2], ya[3]};
    *reinterpret_cast<uint4*>(row + d0 + half) = uint4{yb[0], yb[1], yb[2], yb[3]};
  }
}

// One workgroup per appended token: threads 0..127 copy its key row (4 heads x 256 dims),
// threads 128..255 its value row, 16 bytes each.  With rope_k the key is rotated by its
// position on the way (same arithmetic as rope_qk_kernel): the thread holding dims
// d .. d+7 < r/2 of a head also reads and writes their partners d + r/2 .., the threads
// of dims r/2 .. r-1 write nothing, and dims r .. 255 are copied.
__global__ __launch_bounds__(256) void kv_append_kernel(
    const bf16_t* __restrict__ k_new, const bf16_t* __restrict__ v_new,
    bf16_t* __restrict__ k_cache, bf16_t* __restrict__ v_cache, int cap,
    const int* __restrict__ pos0, int n, int window, int* __restrict__ slots_out, int rope_k,
    RopeTable tab) {
  __shared__ f32x2 cs[kMaxHalfRot];
  const long long tok = blockIdx.x;
  const int b = (int)(tok / n), t = (int)(tok - (long long)b * n);
  const int p = pos0[b] + t;
  int slot;
  bool write;
  if (window == 0) {
    slot = (p >= 0 && p < cap) ? p : -1;
    write = slot >= 0;
  } else {
    slot = p >= 0 ? p % window : -1;
    // Only the last `window` tokens of this call survive; skipping the rest also keeps
    // two workgroups from writing one slot.
    write = slot >= 0 && slot < cap && t >= n - window;
  }
  if (threadIdx.x == 0 && slots_out != nullptr) slots_out[tok] = slot;
  if (!write) return;  // uniform over the workgroup
  const int half = tab.rot_dim >> 1;
  if (rope_k) {
    for (int f = threadIdx.x; f < half; f += 256) {
      float sv, cv;
      sincos_angle(rope_angle(p, tab.inv_freq[f]), &sv, &cv);
      cs[f] = f32x2{cv, sv};
    }
    __syncthreads();
  }
  const int c = threadIdx.x & 127;
  const bool is_v = threadIdx.x >= 128;
  const bf16_t* src = (is_v ? v_new : k_new) + tok * (kHkv * kD) + c * 8;
  bf16_t* dst = (is_v ? v_cache : k_cache) + ((long long)b * cap + slot) * (kHkv * kD) + c * 8;
  const int d0 = (c & 31) * 8;  // first of this thread's 8 dims within its head
  if (!rope_k || is_v || d0 >= 2 * half) {
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
    return;
  }
  if (d0 >= half) return;  // the partner thread writes these dims
  const uint4 xa = *reinterpret_cast<const uint4*>(src);
  const uint4 xb = *reinterpret_cast<const uint4*>(src + half);
  const uint32_t wa[4] = {xa.x, xa.y, xa.z, xa.w};
  const uint32_t wb[4] = {xb.x, xb.y, xb.z, xb.w};
  uint32_t ya[4], yb[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const f32x2 c0 = cs[d0 + 2 * w], c1 = cs[d0 + 2 * w + 1];
    float ya0, yb0, ya1, yb1;
    rope_pair(bf16_lo(wa[w]), bf16_lo(wb[w]), c0.x, c0.y, &ya0, &yb0);
    rope_pair(bf16_hi(wa[w]), bf16_hi(wb[w]), c1.x, c1.y, &ya1, &yb1);
    ya[w] = pack_bf16x2(ya0, ya1);
    yb[w] = pack_bf16x2(yb0, yb1);
  }
  *reinterpret_cast<uint4*>(dst) = uint4{ya[0], ya[1], ya[2], ya[3]};
  *reinterpret_cast<uint4*>(dst + half) = uint4{yb[0], yb[1], yb[2], yb[3]};
}

// 8-bit KV append: one workgroup per token.  The token's key row (rotated first when
// rope_k) and value row are rounded to bf16 as the 16-bit cache would hold them, staged in
// LDS, and each (row, head) of 256 values is quantized with scale = amax / 448 (fp32,
// correctly rounded) to E4M3 codes x / scale (correctly rounded division, clamped to
// +-448, then the hardware's round-to-nearest-even conversion).  A head's 256 values are
// the 32 lanes x 8 values of one half-wave, so its amax is a 5-step lane reduction.
// Caches [B, cap, 4, 256] bytes; scales [B, 4, cap] fp32.
// [T5] §3.2 "Deployment steps and key parameters" (the 1M deployment quantizes the KV
// cache to save memory).
__global__ __launch_bounds__(256) void kv_append_fp8_kernel(
    const bf16_t* __restrict__ k_new, const bf16_t* __restrict__ v_new,
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache, float* __restrict__ k_scale,
    float* __restrict__ v_scale, int cap, const int* __restrict__ pos0, int n, int window,
    int* __restrict__ slots_out, int rope_k, RopeTable tab) {
  __shared__ f32x2 cs[kMaxHalfRot];
  __shared__ __attribute__((aligned(16))) bf16_t row[2][kHkv * kD];
  const long long tok = blockIdx.x;
  const int b = (int)(tok / n), t = (int)(tok - (long long)b * n);
  const int p = pos0[b] + t;
  int slot;
  bool write;
  if (window == 0) {
    slot = (p >= 0 && p < cap) ? p : -1;
    write = slot >= 0;
  } else {
    slot = p >= 0 ? p % window : -1;
    write = slot >= 0 && slot < cap && t >= n - window;
  }
  if (threadIdx.x == 0 && slots_out != nullptr) slots_out[tok] = slot;
  if (!write) return;  // uniform over the workgroup
  const int half = tab.rot_dim >> 1;
  if (rope_k) {
    for (int f = threadIdx.x; f < half; f += 256) {
      float sv, cv;
      sincos_angle(rope_angle(p, tab.inv_freq[f]), &sv, &cv);
      cs[f] = f32x2{cv, sv};
    }
    __syncthreads();
  }
  const int c = threadIdx.x & 127;
  const bool is_v = threadIdx.x >= 128;
  const int head = c >> 5, d0 = (c & 31) * 8;
  const bf16_t* src = (is_v ? v_new : k_new) + tok * (kHkv * kD) + c * 8;
  bf16_t* stage = &row[is_v ? 1 : 0][c * 8];
  // Stage the row as the 16-bit cache would hold it.
  if (!rope_k || is_v || d0 >= 2 * half) {
    *reinterpret_cast<uint4*>(stage) = *reinterpret_cast<const uint4*>(src);
  } else if (d0 < half) {
    const uint4 xa = *reinterpret_cast<const uint4*>(src);
    const uint4 xb = *reinterpret_cast<const uint4*>(src + half);
    const uint32_t wa[4] = {xa.x, xa.y, xa.z, xa.w};
    const uint32_t wb[4] = {xb.x, xb.y, xb.z, xb.w};
    uint32_t ya[4], yb[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f32x2 c0 = cs[d0 + 2 * w], c1 = cs[d0 + 2 * w + 1];
      float ya0, yb0, ya1, yb1;
      rope_pair(bf16_lo(wa[w]), bf16_lo(wb[w]), c0.x, c0.y, &ya0, &yb0);
      rope_pair(bf16_hi(wa[w]), bf16_hi(wb[w]), c1.x, c1.y, &ya1, &yb1);
      ya[w] = pack_bf16x2(ya0, ya1);
      yb[w] = pack_bf16x2(yb0, yb1);
    }
    *reinterpret_cast<uint4*>(stage) = uint4{ya[0], ya[1], ya[2], ya[3]};
    *reinterpret_cast<uint4*>(stage + half) = uint4{yb[0], yb[1], yb[2], yb[3]};
  }
  __syncthreads();
  const uint4 xw = *reinterpret_cast<const uint4*>(stage);
  const uint32_t wv[4] = {xw.x, xw.y, xw.z, xw.w};
  float x[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    x[2 * w] = bf16_lo(wv[w]);
    x[2 * w + 1] = bf16_hi(wv[w]);
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 32));
  const float scale = __fdiv_rn(amax, kE4m3Max);
  uint32_t codes[2] = {0u, 0u};
  if (scale > 0.f) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        y[e] = fminf(fmaxf(__fdiv_rn(x[4 * w + e], scale), -kE4m3Max), kE4m3Max);
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], word, true);
      codes[w] = (uint32_t)word;
    }
  }
  uint8_t* dst = (is_v ? v_cache : k_cache) + ((long long)b * cap + slot) * (kHkv * kD) + c * 8;
  *reinterpret_cast<uint2*>(dst) = uint2{codes[0], codes[1]};
  if ((c & 31) == 0) (is_v ? v_scale : k_scale)[((long long)b * kHkv + head) * cap + slot] = scale;
}

}  // namespace

hipError_t launch_rope_qk(bf16_t* q, bf16_t* k, const int* pos0, int B, int S,
                          const RopeTable& tab, hipStream_t stream) {
  const long long ntok = (long long)B * S;
  const long long grid = (ntok + kRopeTokens - 1) / kRopeTokens;
  hipLaunchKernelGGL(rope_qk_kernel, dim3((unsigned)grid), dim3(kRopeThreads), 0, stream, q, k,
                     pos0, S, ntok, tab);
  return hipGetLastError();
}

hipError_t launch_kv_append(const bf16_t* k_new, const bf16_t* v_new, bf16_t* k_cache,
                            bf16_t* v_cache, int cap, const int* pos0, int B, int n,
                            int window, int* slots_out, const RopeTable* rope_k,
                            hipStream_t stream) {
  const long long grid = (long long)B * n;
  const RopeTable tab = rope_k ? *rope_k : RopeTable{};
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)grid), dim3(256), 0, stream, k_new, v_new,
                     k_cache, v_cache, cap, pos0, n, window, slots_out, rope_k ? 1 : 0, tab);
  return hipGetLastError();
}

}  // namespace hattn

namespace hattn {

hipError_t launch_kv_append_fp8(const bf16_t* k_new, const bf16_t* v_new, uint8_t* k_cache,
                                uint8_t* v_cache, float* k_scale, float* v_scale, int cap,
                                const int* pos0, int B, int n, int window, int* slots_out,
                                const RopeTable* rope_k, hipStream_t stream) {
  const long long grid = (long long)B * n;
  const RopeTable tab = rope_k ? *rope_k : RopeTable{};
  hipLaunchKernelGGL(kv_append_fp8_kernel, dim3((unsigned)grid), dim3(256), 0, stream, k_new,
                     v_new, k_cache, v_cache, k_scale, v_scale, cap, pos0, n, window, slots_out,
                     rope_k ? 1 : 0, tab);
  return hipGetLastError();
}

}  // namespace hattn
