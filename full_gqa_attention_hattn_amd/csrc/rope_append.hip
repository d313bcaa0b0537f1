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
__global__ __launch_bounds__(kRopeThreads) void rope_qk_kernel(
    bf16_t* __restrict__ q, bf16_t* __restrict__ k, const int* __restrict__ pos0, int S,
    long long ntok, RopeTable tab) {
  __shared__ f32x2 cs[kRopeTokens][kMaxHalfRot];
  const int half = tab.rot_dim >> 1;
  const long long tok0 = (long long)blockIdx.x * kRopeTokens;

  for (int e = threadIdx.x; e < kRopeTokens * half; e += kRopeThreads) {
    const int t = e / half, f = e - t * half;
    const long long tok = tok0 + t;
    if (tok < ntok) {
      const int b = (int)(tok / S), s = (int)(tok - (long long)b * S);
      const int p = pos0[b] + s;
      float sv, cv;
      sincos_angle(rope_angle(p, tab.inv_freq[f]), &sv, &cv);
      cs[t][f] = f32x2{cv, sv};
    }
  }
  __syncthreads();

  const int groups = half >> 3;              // 8 pairs per item
  const int per_tok = (kHq + kHkv) * groups;  // heads 0..15 of q, then 4 of k
  for (int e = threadIdx.x; e < kRopeTokens * per_tok; e += kRopeThreads) {
    const int t = e / per_tok;
    const int rem = e - t * per_tok;
    const int hh = rem / groups, gi = rem - hh * groups;
    const long long tok = tok0 + t;
    if (tok >= ntok) continue;
    bf16_t* row;
    if (hh < kHq) {
      if (q == nullptr) continue;
      row = q + (tok * kHq + hh) * kD;
    } else {
      if (k == nullptr) continue;
      row = k + (tok * kHkv + (hh - kHq)) * kD;
    }
    const int d0 = gi * 8;
    uint4 xa = *reinterpret_cast<const uint4*>(row + d0);
    uint4 xb = *reinterpret_cast<const uint4*>(row + d0 + half);
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
