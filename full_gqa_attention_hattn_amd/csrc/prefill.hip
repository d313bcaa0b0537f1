// Flash-style prefill for one hybrid-attention layer on CDNA4 (gfx950).
//
// What it computes (per sequence b, query row i at position p = pos0[b] + i, head h):
//   s_j  = (q_rot . k_j) / 16 over the visible keys j
//          full: 0 <= j <= p          sliding: p - 511 <= j <= p
//   out  = bf16( sigmoid(gate) * sum_j softmax(s)_j v_j ),   lse = ln sum_j exp(s_j)
// with KV head h / 4 for query head h.  [T1] "Hybrid attention" (causal mask on full layers,
// sliding-window causal mask on sliding layers); [T1] "GQA, fused projection and output
// gating" (16 query heads share 4 KV heads; sigmoid gate multiplied into each head's
// output); [T2] "Grouped-query attention"; [T3] "Sliding window 512".
//
// Design (one workgroup = 4 waves = one KV head x 32 query positions):
//   * wave w owns query head 4*kvh + w, so every K/V tile staged in LDS feeds all 4 heads
//     of its group;
//   * S^T = K . Q^T and O^T = V^T . P^T run on v_mfma_f32_32x32x16_bf16 with fp32
//     accumulation: a lane holds one query row's scores, so the online-softmax max/sum
//     need one cross-lane exchange (lane ^ 32) and the rescale of O is lane-local;
//   * P^T goes from the score accumulators to the PV MFMA in registers: V^T is written to
//     LDS with its keys in the order a lane's accumulator holds them;
//   * K and V^T tiles (64 keys) are double-buffered in XOR-swizzled LDS (conflict-free
//     16-byte MFMA operand reads), loaded one tile ahead through registers;
//   * tiles wholly outside the causal / sliding band are never visited; only tiles that
//     straddle the band edge or the diagonal evaluate the element mask;
//   * optional fused Q-RoPE: the workgroup computes cos/sin of its 32 positions once into
//     LDS and each lane rotates its own Q fragment (pairs d, d + r/2 sit in the same lane);
//   * epilogue: 1/l, sigmoid gate, bf16 store, optional fp32 LSE.
#include "hattn_device.h"
#include "hattn_launch.h"

namespace hattn {

namespace {

constexpr int kBQ = 32;                   // query positions per workgroup
constexpr int kBN = 64;                   // keys per tile
constexpr int kThreads = 256;             // 4 waves
constexpr int kKBytes = kBN * kD * 2;     // K tile: 64 rows x 512 B
constexpr int kVBytes = kD * kBN * 2;     // V^T tile: 256 rows x 128 B
constexpr int kStage = kKBytes + kVBytes;
constexpr int kLds = 2 * kStage;
constexpr float kLn2 = 0.69314718055994530942f;

// K tile: key row r, 16-byte block c (dims 8c..8c+7) at r*512 + ((c ^ (r & 7)) << 4).
__device__ __forceinline__ int k_off(int r, int c) { return r * 512 + ((c ^ (r & 7)) << 4); }

// V^T tile: dim row d, 16-byte block c (8 key slots) at d*128 + ((c ^ swz(d)) << 4).
__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }
__device__ __forceinline__ int vt_off(int d, int c) { return d * 128 + ((c ^ vt_swz(d)) << 4); }

// Slot of key kl (0..15) inside its 16-key chunk of a V^T row.  Lane half hh of the score
// accumulator holds, per 16-key chunk, keys 4hh..4hh+3 then 8+4hh..8+4hh+3; those land in
// slots 8hh..8hh+7, which is what that lane half reads as the PV operand.
__device__ __forceinline__ int v_slot(int kl) {
  return ((kl >> 2) & 1) * 8 + (kl >> 3) * 4 + (kl & 3);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

struct TileRegs {
  uint4 k[8];
  uint4 v[8];
};

// Global -> registers for the 64-key tile starting at key0.  Rows at or past `cap` read as
// zero and are never dereferenced.
__device__ __forceinline__ void load_tile(TileRegs& R, const bf16_t* kbase, const bf16_t* vbase,
                                          int key0, int cap, int tid) {
  constexpr long long rs = kHkv * kD;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int item = it * kThreads + tid;  // 2048 16-byte blocks
    const int r = item >> 5, c = item & 31;
    const int key = key0 + r;
    R.k[it] = key < cap ? *reinterpret_cast<const uint4*>(kbase + key * rs + c * 8)
                        : uint4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int item = it * kThreads + tid;  // 512 items of 4 keys x 8 dims
    const int dg = item & 31, kg = item >> 5;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + kg * 4 + r;
      R.v[it * 4 + r] = key < cap ? *reinterpret_cast<const uint4*>(vbase + key * rs + dg * 8)
                                  : uint4{0u, 0u, 0u, 0u};
    }
  }
}

// Registers -> LDS stage: K as is (swizzled), V transposed 4 keys x 8 dims per item.
__device__ __forceinline__ void store_tile(const TileRegs& R, char* kst, char* vst, int tid) {
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int item = it * kThreads + tid;
    const int r = item >> 5, c = item & 31;
    *reinterpret_cast<uint4*>(kst + k_off(r, c)) = R.k[it];
  }
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int item = it * kThreads + tid;
    const int dg = item & 31, kg = item >> 5;
    const int kl0 = kg * 4;
    const int e_idx = (kl0 >> 4) * 16 + v_slot(kl0 & 15);  // 4 consecutive slots
    const int blk = e_idx >> 3, byte = (e_idx & 7) * 2;
    const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&R.v[it * 4 + 0]);
    const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&R.v[it * 4 + 1]);
    const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&R.v[it * 4 + 2]);
    const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&R.v[it * 4 + 3]);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int d = dg * 8 + 2 * w;
      const uint2 lo{__builtin_amdgcn_perm(r1[w], r0[w], 0x05040100u),
                     __builtin_amdgcn_perm(r3[w], r2[w], 0x05040100u)};
      const uint2 hi{__builtin_amdgcn_perm(r1[w], r0[w], 0x07060302u),
                     __builtin_amdgcn_perm(r3[w], r2[w], 0x07060302u)};
      *reinterpret_cast<uint2*>(vst + vt_off(d, blk) + byte) = lo;
      *reinterpret_cast<uint2*>(vst + vt_off(d + 1, blk) + byte) = hi;
    }
  }
}

template <bool kSliding>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc,
                    const bf16_t* __restrict__ vc, int cap, const int* __restrict__ pos0, int B,
                    int Sq, const bf16_t* __restrict__ gate, bf16_t* __restrict__ out,
                    float* __restrict__ lse, int window, int rope_q, RopeTable tab, float sl2,
                    int nqb, int nwork) {
  constexpr int kHalf = kSliding ? 128 : 32;  // rot_dim / 2
  constexpr int kNdc = kHalf / 16;           // Q fragments holding the first rotary half
  __shared__ __attribute__((aligned(16))) char smem[kLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;

  int qb, b, kvh;
  if (kSliding) {
    // Equal work per workgroup: give each XCD (blockIdx % 8) a contiguous run of query
    // blocks so the K/V tiles that neighbouring blocks share stay in that XCD's L2.
    const int per = (int)(gridDim.x >> 3);
    const int logical = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (logical >= nwork) return;
    qb = logical % nqb;
    const int rest = logical / nqb;
    kvh = rest % kHkv;
    b = rest / kHkv;
  } else {
    // Causal: longest rows first; consecutive blocks share a query block, so every XCD
    // sees one KV head and all its workgroups stream the same K/V prefix.
    const int bk = B * kHkv;
    qb = nqb - 1 - (int)(blockIdx.x / bk);
    const int rest = (int)(blockIdx.x % bk);
    kvh = rest % kHkv;
    b = rest / kHkv;
  }
  const int h = kvh * kGroup + w;
  const int i0 = qb * kBQ;
  const int nrows = min(kBQ, Sq - i0);
  const int P0 = pos0[b] + i0;
  const int Plast = P0 + nrows - 1;
  const bool row_ok = n < nrows;
  const int row_i = i0 + (row_ok ? n : 0);
  const int prow = P0 + n;

  // Q^T operand: lane (n, hh) holds dims 16dc + 8hh .. +7 of query row n.
  bf16x8 qf[16];
  {
    const bf16_t* qrow = q + (((long long)b * Sq + row_i) * kHq + h) * kD + 8 * hh;
#pragma unroll
    for (int dc = 0; dc < 16; ++dc) {
      qf[dc] = row_ok ? *reinterpret_cast<const bf16x8*>(qrow + 16 * dc) : bf16x8{};
    }
  }

  if (rope_q) {
    constexpr int kPitch = kHalf + 2;  // f32x2 per row; +16 B breaks LDS bank aliasing
    f32x2* cs = reinterpret_cast<f32x2*>(smem);
    for (int e = tid; e < kBQ * kHalf; e += kThreads) {
      const int r = e / kHalf, f = e - r * kHalf;
      float sv, cv;
      sincos_angle(rope_angle(P0 + r, tab.inv_freq[f]), &sv, &cv);
      cs[r * kPitch + f] = f32x2{cv, sv};
    }
    __syncthreads();
#pragma unroll
    for (int dc = 0; dc < kNdc; ++dc) {
      const f32x2* c8 = cs + n * kPitch + 16 * dc + 8 * hh;
      const bf16x8 xa = qf[dc], xb = qf[dc + kNdc];
      f32x4 ya0, ya1, yb0, yb1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const f32x2 c = c8[e];
        const float a = (float)xa[e], bb = (float)xb[e];
        const float ya = a * c.x - bb * c.y;
        const float yb = bb * c.x + a * c.y;
        if (e < 4) { ya0[e] = ya; yb0[e] = yb; } else { ya1[e - 4] = ya; yb1[e - 4] = yb; }
      }
      const bf16x4 a0 = __builtin_convertvector(ya0, bf16x4), a1 = __builtin_convertvector(ya1, bf16x4);
      const bf16x4 b0 = __builtin_convertvector(yb0, bf16x4), b1 = __builtin_convertvector(yb1, bf16x4);
      qf[dc] = bf16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      qf[dc + kNdc] = bf16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    }
    __syncthreads();  // the cos/sin table shares LDS with the first tile
  }

  const int kmax = min(Plast, cap - 1);
  const int kmin = kSliding ? max(0, P0 - (window - 1)) : 0;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) o[mb] = f32x16{};

  const long long kv_off = ((long long)b * cap * kHkv + kvh) * kD;
  const bf16_t* kbase = kc + kv_off;
  const bf16_t* vbase = vc + kv_off;

  if (kmax >= kmin) {
    const int t_lo = kmin / kBN, t_hi = kmax / kBN;
    TileRegs R;
    load_tile(R, kbase, vbase, t_lo * kBN, cap, tid);
    store_tile(R, smem, smem + kKBytes, tid);
    __syncthreads();
    for (int t = t_lo; t <= t_hi; ++t) {
      const char* kst = smem + ((t - t_lo) & 1) * kStage;
      const char* vst = kst + kKBytes;
      const bool more = t < t_hi;
      if (more) load_tile(R, kbase, vbase, (t + 1) * kBN, cap, tid);

      // S^T[key][query] for keys 0..31 (s0) and 32..63 (s1) of the tile.
      f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
      for (int dc = 0; dc < 16; ++dc) {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(kst + k_off(n, 2 * dc + hh));
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(kst + k_off(32 + n, 2 * dc + hh));
        s0 = mfma32(a0, qf[dc], s0);
        s1 = mfma32(a1, qf[dc], s1);
      }

      // Accumulator element 4i + j of lane half hh is key 8i + 4hh + j (+32 for s1).
      const int key0 = t * kBN;
      const bool whole = (key0 + kBN - 1 <= P0) && (key0 + kBN <= cap) &&
                         (!kSliding || Plast - key0 <= window - 1);
      float mloc = -INFINITY;
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        float a = s0[idx] * sl2, c = s1[idx] * sl2;
        if (!whole) {
          const int j0 = key0 + 8 * (idx >> 2) + 4 * hh + (idx & 3);
          const int j1 = j0 + 32;
          const bool v0 = j0 <= prow && j0 < cap && (!kSliding || prow - j0 <= window - 1);
          const bool v1 = j1 <= prow && j1 < cap && (!kSliding || prow - j1 <= window - 1);
          a = v0 ? a : -INFINITY;
          c = v1 ? c : -INFINITY;
        }
        s0[idx] = a;
        s1[idx] = c;
        mloc = fmaxf(mloc, fmaxf(a, c));
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_new = fmaxf(m_run, mloc);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float rs = 0.f;
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        s0[idx] = fast_exp2(s0[idx] - m_use);
        s1[idx] = fast_exp2(s1[idx] - m_use);
        rs += s0[idx] + s1[idx];
      }
      l_run = l_run * alpha + rs;
      m_run = m_new;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) o[mb] *= alpha;
      }

      // P^T operands, one per 16-key chunk, straight from the accumulators.
      bf16x8 pf[4];
      {
        const f32x4 c0 = {s0[0], s0[1], s0[2], s0[3]}, c1 = {s0[4], s0[5], s0[6], s0[7]};
        const f32x4 c2 = {s0[8], s0[9], s0[10], s0[11]}, c3 = {s0[12], s0[13], s0[14], s0[15]};
        const f32x4 c4 = {s1[0], s1[1], s1[2], s1[3]}, c5 = {s1[4], s1[5], s1[6], s1[7]};
        const f32x4 c6 = {s1[8], s1[9], s1[10], s1[11]}, c7 = {s1[12], s1[13], s1[14], s1[15]};
        const bf16x4 b0 = __builtin_convertvector(c0, bf16x4), b1 = __builtin_convertvector(c1, bf16x4);
        const bf16x4 b2 = __builtin_convertvector(c2, bf16x4), b3 = __builtin_convertvector(c3, bf16x4);
        const bf16x4 b4 = __builtin_convertvector(c4, bf16x4), b5 = __builtin_convertvector(c5, bf16x4);
        const bf16x4 b6 = __builtin_convertvector(c6, bf16x4), b7 = __builtin_convertvector(c7, bf16x4);
        pf[0] = bf16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        pf[1] = bf16x8{b2[0], b2[1], b2[2], b2[3], b3[0], b3[1], b3[2], b3[3]};
        pf[2] = bf16x8{b4[0], b4[1], b4[2], b4[3], b5[0], b5[1], b5[2], b5[3]};
        pf[3] = bf16x8{b6[0], b6[1], b6[2], b6[3], b7[0], b7[1], b7[2], b7[3]};
      }
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vst + vt_off(32 * mb + n, 2 * c + hh));
          o[mb] = mfma32(a, pf[c], o[mb]);
        }
      }

      if (more) {
        char* nk = smem + ((t + 1 - t_lo) & 1) * kStage;
        store_tile(R, nk, nk + kKBytes, tid);
      }
      __syncthreads();
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (row_ok) {
    const long long row = (long long)b * Sq + row_i;
    const float g = bf16_to_f32(gate[row * kHq + h]);
    const float sg = 1.f / (1.f + expf(-g));
    const float f = l_tot > 0.f ? sg / l_tot : 0.f;
    bf16_t* orow = out + (row * kHq + h) * kD + 4 * hh;
    // O^T accumulator element 4i + j of block mb is dim 32mb + 8i + 4hh + j.
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint2 v{pack_bf16x2(o[mb][4 * i] * f, o[mb][4 * i + 1] * f),
                      pack_bf16x2(o[mb][4 * i + 2] * f, o[mb][4 * i + 3] * f)};
        *reinterpret_cast<uint2*>(orow + 32 * mb + 8 * i) = v;
      }
    }
    if (lse != nullptr && hh == 0) {
      lse[row * kHq + h] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_prefill(const bf16_t* q, const bf16_t* k_cache, const bf16_t* v_cache, int cap,
                          const int* pos0, int B, int Sq, const bf16_t* gate, bf16_t* out,
                          float* lse, int window, bool rope_q, const RopeTable& tab,
                          float scale_log2e, hipStream_t stream) {
  const int nqb = (Sq + kBQ - 1) / kBQ;
  const long long nwork = (long long)B * kHkv * nqb;
  if (window > 0) {
    const long long grid = (nwork + 7) / 8 * 8;
    hipLaunchKernelGGL(prefill_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, stream, q,
                       k_cache, v_cache, cap, pos0, B, Sq, gate, out, lse, window, rope_q ? 1 : 0,
                       tab, scale_log2e, nqb, (int)nwork);
  } else {
    hipLaunchKernelGGL(prefill_kernel<false>, dim3((unsigned)nwork), dim3(kThreads), 0, stream, q,
                       k_cache, v_cache, cap, pos0, B, Sq, gate, out, lse, window, rope_q ? 1 : 0,
                       tab, scale_log2e, nqb, (int)nwork);
  }
  return hipGetLastError();
}

}  // namespace hattn
