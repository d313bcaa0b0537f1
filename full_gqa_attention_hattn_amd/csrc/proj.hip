// Projections around one attention layer on bf16 MFMA: the fused QKV + gate projection
// (hidden 2560 -> q 4096, k 1024, v 1024, gate 16) and the output projection (4096 ->
// 2560).  [T1] "GQA, fused projection and output gating": one linear layer whose output
// is sliced in order into q, k and v, and a per-head g_proj gate score; [T4] parameter
// table (hidden 2560) and its quantization section (o_proj).
//
// Both are Y = X W^T with X [T, K] and W [N, K] row-major (the linear-layer layout), so
// both operands are rows with K contiguous.  A workgroup computes one tile
// Y^T[n][t] = sum_k W[n][k] X[t][k] on v_mfma_f32_32x32x16_bf16 (A = W rows, B = X rows),
// each wave a block of 32 x 32 outputs per accumulator.  64-wide K slices of both operands go
// global -> LDS directly (the buffer form of the LDS copy, which keeps the fragment reads'
// LDS waits exact), double-buffered, each 128-byte row with its 16-byte blocks XOR-swizzled
// by (row >> 1) & 7 so that the 16 rows one 16-lane group reads hit 16 different bank
// groups.  Each MFMA of a 16-wide k-step is paired with one fragment read of the next.
//
// Three tile shapes; per call the launcher takes the one with the least estimated time,
// whole rounds of tiles over the CUs times a tile's cost (a partly filled last round costs a
// full one):
//  - 128 x 128, four waves of 64 x 64, two workgroups per CU (64 KiB of LDS each).  The
//    next slice's copies go out at the top of a k-step and one barrier ends it; the other
//    workgroup on the CU covers the wait.  Best below a few thousand tokens.
//  - 192 x 256 (QKV) and 160 x 256 (output), eight waves of 96 x 64 and four of 160 x 64,
//    one workgroup per CU.  At 4096 tokens these make exactly two rounds (the 6144 q/k/v
//    rows; the 16 gate rows then run as a small kernel of their own) and exactly one round.
//    With no second workgroup to cover the barrier the k-step is rotated: the next slice's
//    copies are spread over the first half of its MFMAs, the barrier sits after the first
//    MFMA of the last 16-wide step, and the remaining MFMAs cover the reads of the next
//    slice's first fragments, issued in the order the MFMAs first use them.
// Tiles are ordered so that each XCD works on a band of token tiles across all feature
// tiles (L2 reuse of both operands).  The accumulator holds 4 consecutive output features
// of one token per lane group, stored as 8-byte bf16 runs, each routed to q, k, v, the gate
// logits or Y in the layouts the attention calls take.
#include <atomic>
#include <type_traits>

#include "hattn_device.h"
#include "hattn_launch.h"

namespace hattn {

namespace {

constexpr int kBK = 64;               // K per slice
constexpr int kRowB = 2 * kBK;        // bytes of one row segment
constexpr int kBlk = kRowB / 16;      // 16-byte blocks per row segment
constexpr int kKS = kBK / 16;         // MFMA k-steps per slice
constexpr int kQDim = kHq * kD, kKvDim = kHkv * kD, kQkvDim = kQDim + 2 * kKvDim;
constexpr int kGateRows = kHq;

typedef __attribute__((address_space(3))) void lds_void;

// Row r's 16-byte block b sits at b ^ pswz(r): the 16 rows one 16-lane group reads (at one
// block) then fall on 16 different bank groups (rows r and r ^ 1 use the two halves of the
// banks).
__device__ __forceinline__ int pswz(int r) { return (r >> 1) & 7; }

// One 1 KiB global->LDS copy (16 bytes a lane, at byte offset voff from base).  With
// live == false the buffer range is empty: nothing is read and the LDS bytes are don't-care.
__device__ __forceinline__ void copy_piece(char* dst, const bf16_t* base, bool live, int voff) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(base), (short)0, live ? 0x7fffffff : 0, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 16, voff, 0, 0, 0);
}

// Waits until at most n vector-memory operations of this wave are in flight.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
}

// The same, and every LDS read of this wave has returned.
template <int n>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0070 | (n & 15) | ((n >> 4) << 14));
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Tile shape: a kGN x kGT grid of waves, each owning kAN x kAT blocks of 32 x 32 outputs
// (kAN along the features, kAT along the tokens); kRotate selects the rotated k-step.
template <int kAN_, int kAT_, int kGN_, int kGT_, bool kRotate_>
struct Shape {
  static constexpr int kAN = kAN_, kAT = kAT_, kGN = kGN_, kGT = kGT_;
  static constexpr bool kRotate = kRotate_;
  static constexpr int kWaves = kGN * kGT, kThreads = 64 * kWaves;
  static constexpr int kTN = 32 * kAN * kGN, kTT = 32 * kAT * kGT;
  static constexpr int kWBytes = kTN * kRowB, kXBytes = kTT * kRowB;
  static constexpr int kStageBytes = kWBytes + kXBytes;
  // Copies per slice: kNW 1 KiB pieces of W rows and kNX of X rows per wave.
  static constexpr int kNW = kWBytes / 1024 / kWaves, kNX = kXBytes / 1024 / kWaves;
  static_assert(kNW * 1024 * kWaves == kWBytes && kNX * 1024 * kWaves == kXBytes,
                "slice copies split evenly over the waves");
};
using TileA = Shape<2, 2, 2, 2, false>;  // 128 x 128
using TileQ = Shape<3, 2, 2, 4, true>;   // 192 x 256, q/k/v rows
using TileO = Shape<5, 2, 1, 4, true>;   // 160 x 256

// kFused: 0 = plain Y [T, N]; 1 = the QKV + gate projection (features >= 6144 are gate rows).
template <int kFused, class S>
__global__ __launch_bounds__(S::kThreads) void proj_kernel(
    const bf16_t* __restrict__ x, int T, int K, const bf16_t* __restrict__ w,
    const bf16_t* __restrict__ w_gate, int N, bf16_t* __restrict__ y0, bf16_t* __restrict__ y1,
    bf16_t* __restrict__ y2, bf16_t* __restrict__ y3, int nN, int nT, int gN) {
  constexpr int kAN = S::kAN, kAT = S::kAT, kGN = S::kGN, kWaves = S::kWaves;
  constexpr int kTN = S::kTN, kTT = S::kTT;
  constexpr int kF = kAN + kAT, kM = kAN * kAT;  // fragments and MFMAs per k-step
  constexpr int kNW = S::kNW, kNC = S::kNW + S::kNX;
  static_assert(!kFused || kQkvDim % kTN == 0, "no tile spans both q/k/v and gate rows");
  __shared__ __attribute__((aligned(1024))) char smem[2 * S::kStageBytes];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wn = wv % kGN, wt = wv / kGN;
  // Tile order.  Workgroup i runs on XCD i % 8.  With gN > 0 the 8 XCDs split the tiles
  // into gN feature bands x 8 / gN token bands, and XCD x walks its band with the feature
  // tile varying fastest, so each XCD's L2 fetches only its bands' slices of W and X (the
  // launcher picks gN for the least fetched bytes).  Otherwise, with 8+ token tiles, XCD x
  // owns a contiguous band of token tiles across all feature tiles.
  int nb, tb;
  {
    const int id = (int)blockIdx.x;
    if (gN > 0) {
      const int xcd = id & 7, local = id >> 3;
      const int bn = nN / gN, bt = nT / (8 / gN);
      if (local >= bn * bt) return;
      nb = (xcd % gN) * bn + local % bn;
      tb = (xcd / gN) * bt + local / bn;
    } else if (nT >= 8) {
      const int xcd = id & 7, local = id >> 3;
      const int per = (nT + 7) >> 3;
      const int t_lo = xcd * per;
      const int t_cnt = max(0, min(per, nT - t_lo));
      if (local >= nN * t_cnt) return;
      nb = local / t_cnt;
      tb = t_lo + local % t_cnt;
    } else {
      if (id >= nN * nT) return;
      nb = id % nN;
      tb = id / nN;
    }
  }
  const int n_tile = nb * kTN, t_tile = tb * kTT;

  // This tile's weight rows (a tile lies inside the q/k/v rows or inside the gate rows);
  // rows past the last read the last one.
  const bool gate_tile = kFused && n_tile >= kQkvDim;
  const bf16_t* wbase = gate_tile ? w_gate : w;
  const int wrow0 = gate_tile ? n_tile - kQkvDim : n_tile;
  const int wlast = gate_tile ? kGateRows - 1 : (kFused ? kQkvDim - 1 : N - 1);

  f32x16 acc[kAN][kAT];
#pragma unroll
  for (int a = 0; a < kAN; ++a)
#pragma unroll
    for (int b = 0; b < kAT; ++b) acc[a][b] = f32x16{};

  // Copy c of a slice is 1 KiB piece j = kWaves i + wv of the W rows (c = i < kNW) or of
  // the X rows (c = kNW + i).  Lane l of piece j lands at row (1024 j + 16 l) / kRowB,
  // physical block l % kBlk, so it fetches the logical block (l % kBlk) ^ pswz(row).
  const int nk = K / kBK;
  int voff[kNC];
#pragma unroll
  for (int c = 0; c < kNC; ++c) {
    const bool wm = c < kNW;
    const int j = kWaves * (wm ? c : c - kNW) + wv;
    const int row = (1024 * j + 16 * lane) / kRowB;
    const int lb = (lane % kBlk) ^ pswz(row);
    const int r = wm ? min(wrow0 + row, wlast) - wrow0 : min(t_tile + row, T - 1) - t_tile;
    voff[c] = r * K * 2 + 16 * lb;
  }
  const bf16_t* wsl = wbase + (long long)wrow0 * K;
  const bf16_t* xsl = x + (long long)t_tile * K;
  // Copy c of slice kt into stage s.  Slices past the end go out with an empty range, so
  // every k-step issues the same copies and the wait counts stay fixed.
  auto copy = [&](int s, int kt, int c) {
    const bool wm = c < kNW;
    const int j = kWaves * (wm ? c : c - kNW) + wv;
    copy_piece(smem + s * S::kStageBytes + (wm ? 0 : S::kWBytes) + j * 1024,
               (wm ? wsl : xsl) + min(kt, nk - 1) * kBK, kt < nk, voff[c]);
  };
  const int r32 = lane & 31, hk = lane >> 5;
  // Fragment f of k-step kk of the slice at stage base ws: f < kAN are W rows (a), the rest
  // X rows (b).
  auto frag = [&](const char* ws, int kk, int f) {
    const int lb = 2 * kk + hk;
    const int row = f < kAN ? 32 * kAN * wn + 32 * f + r32 : 32 * kAT * wt + 32 * (f - kAN) + r32;
    const char* base = f < kAN ? ws : ws + S::kWBytes;
    return *reinterpret_cast<const bf16x8*>(base + row * kRowB + ((lb ^ pswz(row)) << 4));
  };

#pragma unroll
  for (int c = 0; c < kNC; ++c) copy(0, 0, c);
  wait_vm<0>();
  __syncthreads();

  if constexpr (!S::kRotate) {
    static_assert(kM >= kF, "one fragment read per MFMA covers the next k-step");
    for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
      for (int c = 0; c < kNC; ++c) copy((kt + 1) & 1, kt + 1, c);
      const char* ws = smem + (kt & 1) * S::kStageBytes;
      bf16x8 cur[kF], nxt[kF];
#pragma unroll
      for (int f = 0; f < kF; ++f) cur[f] = frag(ws, 0, f);
#pragma unroll
      for (int kk = 0; kk < kKS; ++kk) {
#pragma unroll
        for (int j = 0; j < kM; ++j) {
          const int a = j / kAT, b = j % kAT;
          acc[a][b] = mfma32(cur[a], cur[kAN + b], acc[a][b]);
          if (kk + 1 < kKS && j < kF) nxt[j] = frag(ws, kk + 1, j);
        }
#pragma unroll
        for (int f = 0; f < kF; ++f) cur[f] = nxt[f];
      }
      __builtin_amdgcn_sched_group_barrier(0x100, kF, 0);
#pragma unroll
      for (int kk = 0; kk + 1 < kKS; ++kk)
#pragma unroll
        for (int j = 0; j < kM; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (j < kF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      __builtin_amdgcn_sched_group_barrier(0x008, kM, 0);
      __builtin_amdgcn_sched_barrier(0);  // the MFMAs stay ahead of the wait and barrier
      wait_vm<0>();
      __syncthreads();
    }
  } else {
    // Copy c of the next slice follows MFMA slot c * kSpan / kNC of the first half of the
    // k-step; all of them precede the barrier that waits for them.
    constexpr int kSpan = kKS * kM / 2;
    static_assert((kNC - 1) * kSpan / kNC < (kKS - 1) * kM, "copies precede the barrier");
    // Reads in the order the next step's MFMAs first use the fragments: a0, b0 .. b_last,
    // a1 .. a_last.
    auto rd = [](int i) { return i == 0 ? 0 : i <= kAT ? kAN + i - 1 : i - kAT; };
    bf16x8 cur[kF], nxt[kF];
#pragma unroll
    for (int f = 0; f < kF; ++f) cur[f] = frag(smem, 0, f);
    auto kstep = [&](int kt, auto last_tag) {
      constexpr bool kLast = decltype(last_tag)::value;
      const char* ws = smem + (kt & 1) * S::kStageBytes;
      const char* wnext = smem + ((kt + 1) & 1) * S::kStageBytes;
#pragma unroll
      for (int kk = 0; kk < kKS; ++kk) {
        const bool tail = kk + 1 == kKS;
#pragma unroll
        for (int j = 0; j < kM; ++j) {
          const int a = j / kAT, b = j % kAT;
          acc[a][b] = mfma32(cur[a], cur[kAN + b], acc[a][b]);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (!tail) {
            if (j < kF) {
              nxt[rd(j)] = frag(ws, kk + 1, rd(j));
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
          } else if (!kLast) {
            if (j == 0) {
              // The next slice has landed and no wave still reads the stage the next
              // k-step's copies will overwrite.
              __builtin_amdgcn_sched_barrier(0);
              wait_vm_lgkm0<0>();
              __syncthreads();
            } else if (j - 1 < kF) {
              nxt[rd(j - 1)] = frag(wnext, 0, rd(j - 1));
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
          }
#pragma unroll
          for (int c = 0; c < kNC; ++c)
            if (!kLast && c * kSpan / kNC == kk * kM + j) {
              copy((kt + 1) & 1, kt + 1, c);
              __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        }
        if (!tail) {
#pragma unroll
          for (int j = kM; j < kF; ++j) nxt[rd(j)] = frag(ws, kk + 1, rd(j));
        } else if (!kLast) {
#pragma unroll
          for (int f = kM - 1; f < kF; ++f) nxt[rd(f)] = frag(wnext, 0, rd(f));
        }
#pragma unroll
        for (int f = 0; f < kF; ++f) cur[f] = nxt[f];
      }
    };
    for (int kt = 0; kt + 1 < nk; ++kt) kstep(kt, std::false_type{});
    kstep(nk - 1, std::true_type{});
  }
  wait_vm<0>();  // no copy may still be writing this workgroup's LDS when it exits

  // acc[a][b] element 4i + j: feature 32 kAN wn + 32a + 8i + 4hk + j, token
  // 32 kAT wt + 32b + r32.  The lanes hk = 0 and 1 of a token (r32 and r32 + 32) hold
  // alternate 4-feature pieces; v_permlane32_swap trades one piece of each pair (i = 2ip,
  // 2ip + 1) between them, so lane hk ends with features 16ip + 8hk .. + 7 of the block and
  // stores 16 contiguous bytes.  Each run of 8 features goes to q, k, v, the gate logits or
  // Y (N and the q/k/v/gate boundaries are multiples of 8).
#pragma unroll
  for (int b = 0; b < kAT; ++b) {
    const int t = t_tile + 32 * kAT * wt + 32 * b + r32;
#pragma unroll
    for (int a = 0; a < kAN; ++a)
#pragma unroll
      for (int ip = 0; ip < 2; ++ip) {
        const int e = 8 * ip;
        const uint32_t a0 = pack_bf16x2(acc[a][b][e], acc[a][b][e + 1]);
        const uint32_t a1 = pack_bf16x2(acc[a][b][e + 2], acc[a][b][e + 3]);
        const uint32_t c0 = pack_bf16x2(acc[a][b][e + 4], acc[a][b][e + 5]);
        const uint32_t c1 = pack_bf16x2(acc[a][b][e + 6], acc[a][b][e + 7]);
        // Upper lanes of the first operand trade with lower lanes of the second (all lanes
        // take part; only valid tokens and features are stored).
        const auto s0 = __builtin_amdgcn_permlane32_swap(a0, c0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(a1, c1, false, false);
        const int f = n_tile + 32 * kAN * wn + 32 * a + 16 * ip + 8 * hk;
        if (t >= T || f >= N) continue;
        bf16_t* dst = y0;
        int col = f, ld = N;
        if (kFused) {
          if (f < kQDim) { ld = kQDim; }
          else if (f < kQDim + kKvDim) { dst = y1; col = f - kQDim; ld = kKvDim; }
          else if (f < kQkvDim) { dst = y2; col = f - kQDim - kKvDim; ld = kKvDim; }
          else { dst = y3; col = f - kQkvDim; ld = kGateRows; }
        }
        *reinterpret_cast<uint4*>(dst + (long long)t * ld + col) =
            uint4{s0[0], s1[0], s0[1], s1[1]};
      }
  }
}

// Small T (decode steps, T <= 32), and the 16 gate rows next to the 192 x 256 tiles: the
// work is split by output feature, token block and K instead.  A workgroup owns 16 features
// of up to 32 tokens; wave w of its kKW takes the w-th K range and runs
// v_mfma_f32_16x16x32_bf16 with A = 16 weight rows and B = up to 16 tokens per block, both
// fragments loaded straight from global memory (16 bytes per lane, kUnroll k-steps in
// flight).  The kKW partial tiles are summed through LDS and wave 0 stores them.
constexpr int kSmallRows = 16;
constexpr int kSmallMaxT = 32;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int kFused, int kTB, int kKW = 4, int kUnroll = 4>
__global__ __launch_bounds__(64 * kKW) void proj_small_kernel(
    const bf16_t* __restrict__ x, int T, int K, const bf16_t* __restrict__ w,
    const bf16_t* __restrict__ w_gate, int N, bf16_t* __restrict__ y0, bf16_t* __restrict__ y1,
    bf16_t* __restrict__ y2, bf16_t* __restrict__ y3, int n_base) {
  __shared__ f32x4 red[kKW][kTB][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  // Grid: x = token blocks (up to 2^31 - 1 of them), y = 16-feature blocks.
  const int n0 = n_base + blockIdx.y * kSmallRows;
  const int t0 = blockIdx.x * 16 * kTB;  // this workgroup's tokens: t0 .. t0 + 16 kTB - 1
  x += (long long)t0 * K;
  T -= t0;
  const bf16_t* wbase = w;
  int wrow = n0;
  bf16_t* dst = y0;
  int dcol0 = n0, dld = N;
  if (kFused) {
    if (n0 >= kQkvDim) { wbase = w_gate; wrow = n0 - kQkvDim; dst = y3; dcol0 = n0 - kQkvDim; dld = kGateRows; }
    else if (n0 < kQDim) { dcol0 = n0; dld = kQDim; }
    else if (n0 < kQDim + kKvDim) { dst = y1; dcol0 = n0 - kQDim; dld = kKvDim; }
    else { dst = y2; dcol0 = n0 - kQDim - kKvDim; dld = kKvDim; }
  }
  const int r16 = lane & 15, kg = lane >> 4;   // fragment row / column and k-group
  const int kq = K / kKW;                      // this wave's K range
  const bf16_t* wr = wbase + (long long)(wrow + r16) * K + wv * kq + 8 * kg;
  const bf16_t* xr[kTB];
#pragma unroll
  for (int tb = 0; tb < kTB; ++tb)
    xr[tb] = x + (long long)min(16 * tb + r16, T - 1) * K + wv * kq + 8 * kg;
  f32x4 acc[kTB];
#pragma unroll
  for (int tb = 0; tb < kTB; ++tb) acc[tb] = f32x4{};
  for (int k = 0; k < kq; k += 32 * kUnroll) {
    bf16x8 a[kUnroll], b[kUnroll][kTB];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      a[u] = *reinterpret_cast<const bf16x8*>(wr + k + 32 * u);
#pragma unroll
      for (int tb = 0; tb < kTB; ++tb) b[u][tb] = *reinterpret_cast<const bf16x8*>(xr[tb] + k + 32 * u);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int tb = 0; tb < kTB; ++tb) acc[tb] = mfma16(a[u], b[u][tb], acc[tb]);
  }
#pragma unroll
  for (int tb = 0; tb < kTB; ++tb) red[wv][tb][lane] = acc[tb];
  __syncthreads();
  if (wv != 0) return;
  // acc element j: feature n0 + 4 kg + j, token 16 tb + r16.
#pragma unroll
  for (int tb = 0; tb < kTB; ++tb) {
    f32x4 v = red[0][tb][lane];
#pragma unroll
    for (int i = 1; i < kKW; ++i) v += red[i][tb][lane];
    const int t = 16 * tb + r16;
    if (t >= T) continue;
    const uint2 o{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *reinterpret_cast<uint2*>(dst + (long long)(t0 + t) * dld + dcol0 + 4 * kg) = o;
  }
}

// Features n_base .. n_base + rows - 1 (a multiple of 16) of all T <= 32 tokens.
template <int kFused>
hipError_t launch_small(const bf16_t* x, int T, int K, const bf16_t* w, const bf16_t* w_gate,
                        int N, bf16_t* y0, bf16_t* y1, bf16_t* y2, bf16_t* y3, int n_base,
                        int rows, hipStream_t stream) {
  const dim3 grid(1, (unsigned)(rows / kSmallRows));
  if (T <= 16)
    hipLaunchKernelGGL((proj_small_kernel<kFused, 1>), grid, dim3(256), 0, stream, x, T, K, w,
                       w_gate, N, y0, y1, y2, y3, n_base);
  else
    hipLaunchKernelGGL((proj_small_kernel<kFused, 2>), grid, dim3(256), 0, stream, x, T, K, w,
                       w_gate, N, y0, y1, y2, y3, n_base);
  return hipGetLastError();
}

// The 16 gate rows of all T tokens: a workgroup per 16 tokens, whose 8 waves split K = 2560
// into ranges of 320 and issue all their loads at once (the kernel streams X once and is
// bound by load latency).
hipError_t launch_gate_rows(const bf16_t* x, int T, const bf16_t* w_gate, bf16_t* gate,
                            hipStream_t stream) {
  constexpr int kKW = 8, kUnroll = kProjHidden / kKW / 32;
  static_assert(kUnroll * 32 * kKW == kProjHidden, "K splits into whole 32-wide steps");
  hipLaunchKernelGGL((proj_small_kernel<1, 1, kKW, kUnroll>), dim3((unsigned)((T + 15) / 16)),
                     dim3(64 * kKW), 0, stream, x, T, kProjHidden, nullptr, w_gate,
                     kQkvDim + kGateRows, nullptr, nullptr, nullptr, gate, kQkvDim);
  return hipGetLastError();
}

// The XCD split for nN x nT tiles of tn x tt: the gN in {1, 2, 4, 8} dividing nN (with
// 8 / gN dividing nT) that fetches the fewest bytes, W / gN + X / (8 / gN) per XCD; 0 when
// none divides (then the token banding below is used).
int xcd_split(int nN, int nT, int tn, int tt, int K) {
  int best = 0;
  double best_bytes = 0.0;
  for (int g = 1; g <= 8; g *= 2) {
    if (nN % g != 0 || nT % (8 / g) != 0) continue;
    const double bytes = (double)nN * tn * K / g + (double)nT * tt * K / (8 / g);
    if (best == 0 || bytes < best_bytes) { best = g; best_bytes = bytes; }
  }
  return best;
}

// Workgroups for nN x nT tiles: every tile once with an XCD split, else 8 bands of
// ceil(nT / 8) token tiles (8+ token tiles) or one per tile.
long long grid_size(int nN, int nT, int gN) {
  if (gN > 0) return (long long)nN * nT;
  return nT >= 8 ? 8LL * nN * ((nT + 7) / 8) : (long long)nN * nT;
}

template <int kFused, class S>
hipError_t launch_tiles(const bf16_t* x, int T, int K, const bf16_t* w, const bf16_t* w_gate,
                        int N, bf16_t* y0, bf16_t* y1, bf16_t* y2, bf16_t* y3,
                        hipStream_t stream) {
  if (N % 8 != 0) return hipErrorInvalidValue;  // the epilogue stores runs of 8 features
  const int nN = (N + S::kTN - 1) / S::kTN, nT = (T + S::kTT - 1) / S::kTT;
  const int gN = xcd_split(nN, nT, S::kTN, S::kTT, K);
  hipLaunchKernelGGL((proj_kernel<kFused, S>), dim3((unsigned)grid_size(nN, nT, gN)),
                     dim3(S::kThreads), 0, stream, x, T, K, w, w_gate, N, y0, y1, y2, y3, nN, nT,
                     gN);
  return hipGetLastError();
}

// Compute units of the current device (cached per device).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Estimated time of a tile shape (arbitrary units): the rounds of tiles the busiest CU runs
// times a tile's area over the shape's measured throughput per CU (TFLOP/s per CU on the
// 4096-token projections: 4.1 for 128 x 128 with two workgroups resident, 3.8 for 192 x 256,
// 4.0 for 160 x 256).
template <class S>
double tile_cost(int N, int T, int cus, double rate) {
  const long long tiles = (long long)((N + S::kTN - 1) / S::kTN) * ((T + S::kTT - 1) / S::kTT);
  return (double)((tiles + cus - 1) / cus) * S::kTN * S::kTT / rate;
}

}  // namespace

hipError_t launch_qkv_proj(const bf16_t* x, int T, const bf16_t* w_qkv, const bf16_t* w_gate,
                           bf16_t* q, bf16_t* k, bf16_t* v, bf16_t* gate, hipStream_t stream) {
  const int N = kQkvDim + kGateRows;
  if (T <= kSmallMaxT)
    return launch_small<1>(x, T, kProjHidden, w_qkv, w_gate, N, q, k, v, gate, 0, N, stream);
  const int cus = cu_count();
  if (tile_cost<TileQ>(kQkvDim, T, cus, 3.8) < tile_cost<TileA>(N, T, cus, 4.1)) {
    // The 6144 q/k/v rows on 192 x 256 tiles, the 16 gate rows on the small kernel.
    const hipError_t e = launch_gate_rows(x, T, w_gate, gate, stream);
    if (e != hipSuccess) return e;
    return launch_tiles<1, TileQ>(x, T, kProjHidden, w_qkv, w_gate, kQkvDim, q, k, v, gate,
                                  stream);
  }
  return launch_tiles<1, TileA>(x, T, kProjHidden, w_qkv, w_gate, N, q, k, v, gate, stream);
}

hipError_t launch_o_proj(const bf16_t* a, int T, const bf16_t* w_o, bf16_t* y,
                         hipStream_t stream) {
  if (T <= kSmallMaxT)
    return launch_small<0>(a, T, kQDim, w_o, nullptr, kProjHidden, y, nullptr, nullptr, nullptr,
                           0, kProjHidden, stream);
  const int cus = cu_count();
  if (tile_cost<TileO>(kProjHidden, T, cus, 4.0) < tile_cost<TileA>(kProjHidden, T, cus, 4.1))
    return launch_tiles<0, TileO>(a, T, kQDim, w_o, nullptr, kProjHidden, y, nullptr, nullptr,
                                  nullptr, stream);
  return launch_tiles<0, TileA>(a, T, kQDim, w_o, nullptr, kProjHidden, y, nullptr, nullptr,
                                nullptr, stream);
}

}  // namespace hattn
