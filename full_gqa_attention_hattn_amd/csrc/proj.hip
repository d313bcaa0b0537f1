// Projections around one attention layer on bf16 MFMA: the fused QKV + gate projection
// (hidden 2560 -> q 4096, k 1024, v 1024, gate 16) and the output projection (4096 ->
// 2560).  [T1] "GQA, fused projection and output gating": one linear layer whose output
// is sliced in order into q, k and v, and a per-head g_proj gate score; [T4] parameter
// table (hidden 2560) and its quantization section (o_proj).
//
// Both are Y = X W^T with X [T, K] and W [N, K] row-major (the linear-layer layout), so
// both operands are rows with K contiguous.  A workgroup computes the 128 x 128 tile
// Y^T[n][t] = sum_k W[n][k] X[t][k] on v_mfma_f32_32x32x16_bf16 (A = W rows, B = X rows),
// four waves of 64 x 64.  64-wide K slices of both operands go global -> LDS directly (the
// buffer form of the LDS copy, which keeps the fragment reads' LDS waits exact),
// double-buffered, each 128-byte row with its 16-byte blocks XOR-swizzled by (row >> 1) & 7
// so that the 16 rows one 16-lane group reads hit 16 different bank groups.  Each MFMA of a 16-wide k-step is paired with one fragment read
// of the next k-step.  Tiles are ordered so that each XCD works on a band of token tiles
// across all feature tiles (L2 reuse of both operands; +16% on the 4096-token QKV case).  The accumulator holds 4 consecutive output features of one
// token per lane group, stored as 8-byte bf16 runs.  The fused projection's epilogue writes
// each 128-feature tile straight into q, k, v or the gate logits (tile edges fall on the
// slice boundaries), in the layouts the attention calls take.
#include "hattn_device.h"
#include "hattn_launch.h"

namespace hattn {

namespace {

constexpr int kTile = 128;            // output features and tokens per workgroup
constexpr int kBK = 64;               // K per stage
constexpr int kStages = 2;            // K slices resident in LDS (measured: 3-5 slower)
constexpr int kRowB = kBK * 2;        // bytes of one row segment
constexpr int kBlk = kRowB / 16;      // 16-byte blocks per row segment
constexpr int kTileBytes = kTile * kBK * 2;
constexpr int kLoadsPerSlice = kTileBytes / 1024 / 4;  // copy instructions per wave per slice
constexpr int kQDim = kHq * kD, kKvDim = kHkv * kD, kQkvDim = kQDim + 2 * kKvDim;
constexpr int kGateRows = kHq;

typedef __attribute__((address_space(3))) void lds_void;

// Row r's 16-byte block b sits at b ^ pswz(r): the 16 rows one 16-lane group reads (at one
// block) then fall on 16 different bank groups.
__device__ __forceinline__ int pswz(int r) { return kBlk == 8 ? (r >> 1) & 7 : (r >> 2) & 3; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Rows row0 .. row0 + 127 (rows past `last` read row `last`), K k0 .. k0 + kBK - 1 of a
// row-major [rows, K] matrix into LDS with the buffer form of the global->LDS copy.  The
// slice is kTileBytes / 1024 instructions of 1 KiB; wave w issues its kLoadsPerSlice.
// Lane l of instruction j lands at row (1024 j + 16 l) / kRowB, physical block l % kBlk,
// so it fetches the logical block (l % kBlk) ^ pswz(row).
__device__ __forceinline__ void load_slice(char* dst, const bf16_t* base, long long ld, int row0,
                                           int last, int k0, int w, int lane) {
  const __amdgpu_buffer_rsrc_t rs = rsrc_of(base + (long long)row0 * ld + k0);
#pragma unroll
  for (int i = 0; i < kLoadsPerSlice; ++i) {
    const int j = kLoadsPerSlice * w + i;
    const int row = (1024 * j + 16 * lane) / kRowB;
    const int lb = (lane % kBlk) ^ pswz(row);
    const int r = min(row0 + row, last) - row0;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + j * 1024), 16,
                                             (int)((long long)r * ld * 2 + 16 * lb), 0, 0, 0);
  }
}

// kFused: 0 = plain Y [T, N]; 1 = the QKV + gate projection (N = 6144 + 16).
template <int kFused>
__global__ __launch_bounds__(256) void proj_kernel(const bf16_t* __restrict__ x, int T, int K,
                                                   const bf16_t* __restrict__ w,
                                                   const bf16_t* __restrict__ w_gate, int N,
                                                   bf16_t* __restrict__ y0, bf16_t* __restrict__ y1,
                                                   bf16_t* __restrict__ y2,
                                                   bf16_t* __restrict__ y3, int nN, int nT) {
  __shared__ __attribute__((aligned(1024))) char smem[kStages * 2 * kTileBytes];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wn = wv & 1, wt = wv >> 1;
  // Tile order: with 8+ token tiles, XCD x (blockIdx % 8) owns a contiguous band of token
  // tiles and walks all feature tiles across it, so the workgroups resident on one XCD
  // share their X and W slices in its L2.
  int nb, tb;
  {
    const int id = (int)blockIdx.x;
    if (nT >= 8) {
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
  const int n_tile = nb * kTile, t_tile = tb * kTile;

  // This tile's weight rows, and where its outputs go.
  const bf16_t* wbase = w;
  int wrow0 = n_tile, wlast = N - 1;
  bf16_t* dst = y0;
  int dcol0 = n_tile, dld = N, dcols = N - n_tile;
  if (kFused) {
    if (n_tile >= kQkvDim) {
      wbase = w_gate; wrow0 = n_tile - kQkvDim; wlast = kGateRows - 1;
      dst = y3; dcol0 = n_tile - kQkvDim; dld = kGateRows; dcols = kGateRows - dcol0;
    } else {
      wlast = kQkvDim - 1;
      if (n_tile < kQDim) { dst = y0; dcol0 = n_tile; dld = kQDim; }
      else if (n_tile < kQDim + kKvDim) { dst = y1; dcol0 = n_tile - kQDim; dld = kKvDim; }
      else { dst = y2; dcol0 = n_tile - kQDim - kKvDim; dld = kKvDim; }
      dcols = kTile;
    }
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  const int nk = K / kBK;
  auto load_stage = [&](int s, int kt) {
    char* st = smem + s * 2 * kTileBytes;
    load_slice(st, wbase, K, wrow0, wlast, kt * kBK, wv, lane);
    load_slice(st + kTileBytes, x, K, t_tile, T - 1, kt * kBK, wv, lane);
  };
  // Stages 0 .. kStages - 2 in flight; stage kt + kStages - 1 is issued while kt computes.
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i)
    if (i < nk) load_stage(i, i);
  // Wait until slice `need` has landed: the slices issued after it may stay in flight.
  // Slices 0 .. min(nk - 1, need + kStages - 2) have been issued when this runs.
  static_assert(kStages >= 2 && kStages <= 5, "wait_slice covers up to 3 later slices");
  auto wait_slice = [&](int need) {
    const int after = min(nk - 1, need + kStages - 2) - need;  // issued later than `need`
    constexpr int L = 2 * kLoadsPerSlice;
    if (after >= kStages - 2) wait_vm<(kStages - 2) * L>();
    else if (after == 2) wait_vm<2 * L>();
    else if (after == 1) wait_vm<L>();
    else wait_vm<0>();
  };
  wait_slice(0);
  __syncthreads();

  const int r32 = lane & 31, hk = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + kStages - 1 < nk) load_stage((kt + kStages - 1) % kStages, kt + kStages - 1);
    const char* ws = smem + (kt % kStages) * 2 * kTileBytes;
    const char* xs = ws + kTileBytes;
    // Fragment f of k-step kk: f = 0, 1 are W rows (a), f = 2, 3 are X rows (b).  Each MFMA
    // of k-step kk is paired with one read of k-step kk + 1, so reads run a k-step ahead.
    auto frag = [&](int kk, int f) {
      const int lb = 2 * kk + hk;
      const int row = f < 2 ? 64 * wn + 32 * f + r32 : 64 * wt + 32 * (f - 2) + r32;
      const char* base = f < 2 ? ws : xs;
      return *reinterpret_cast<const bf16x8*>(base + row * kRowB + ((lb ^ pswz(row)) << 4));
    };
    bf16x8 cur[4], nxt[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) cur[f] = frag(0, f);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int a = j >> 1, b = j & 1;
        acc[a][b] = mfma32(cur[a], cur[2 + b], acc[a][b]);
        if (kk + 1 < kBK / 16) nxt[j] = frag(kk + 1, j);
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) cur[f] = nxt[f];
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 4 * (kBK / 16) - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    if (kt + 1 < nk) wait_slice(kt + 1);
    __syncthreads();
  }

  // acc[a][b] element 4i + j: feature 64wn + 32a + 8i + 4hk + j, token 64wt + 32b + r32.
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int t = t_tile + 64 * wt + 32 * b + r32;
    if (t >= T) continue;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 64 * wn + 32 * a + 8 * i + 4 * hk;  // column within the tile
        if (c >= dcols) continue;
        const uint2 v{pack_bf16x2(acc[a][b][4 * i], acc[a][b][4 * i + 1]),
                      pack_bf16x2(acc[a][b][4 * i + 2], acc[a][b][4 * i + 3])};
        *reinterpret_cast<uint2*>(dst + (long long)t * dld + dcol0 + c) = v;
      }
  }
}

// Small T (decode steps, T <= 32): the weights dominate, so the work is split by output
// feature and K instead.  A workgroup owns 16 features; wave w takes K quarter w and runs
// v_mfma_f32_16x16x32_bf16 with A = 16 weight rows and B = up to 16 tokens per block, both
// fragments loaded straight from global memory (16 bytes per lane, 4 k-steps in flight).
// The four partial tiles are summed through LDS and wave 0 stores them.
constexpr int kSmallRows = 16;
constexpr int kSmallMaxT = 32;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int kFused, int kTB>
__global__ __launch_bounds__(256) void proj_small_kernel(
    const bf16_t* __restrict__ x, int T, int K, const bf16_t* __restrict__ w,
    const bf16_t* __restrict__ w_gate, int N, bf16_t* __restrict__ y0, bf16_t* __restrict__ y1,
    bf16_t* __restrict__ y2, bf16_t* __restrict__ y3) {
  __shared__ f32x4 red[4][kTB][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n0 = blockIdx.x * kSmallRows;
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
  const int kq = K / 4;                        // this wave's K range
  const bf16_t* wr = wbase + (long long)(wrow + r16) * K + wv * kq + 8 * kg;
  const bf16_t* xr[kTB];
#pragma unroll
  for (int tb = 0; tb < kTB; ++tb)
    xr[tb] = x + (long long)min(16 * tb + r16, T - 1) * K + wv * kq + 8 * kg;
  f32x4 acc[kTB];
#pragma unroll
  for (int tb = 0; tb < kTB; ++tb) acc[tb] = f32x4{};
  constexpr int kUnroll = 4;
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
    const f32x4 v = red[0][tb][lane] + red[1][tb][lane] + red[2][tb][lane] + red[3][tb][lane];
    const int t = 16 * tb + r16;
    if (t >= T) continue;
    const uint2 o{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *reinterpret_cast<uint2*>(dst + (long long)t * dld + dcol0 + 4 * kg) = o;
  }
}

template <int kFused>
hipError_t launch_small(const bf16_t* x, int T, int K, const bf16_t* w, const bf16_t* w_gate,
                        int N, bf16_t* y0, bf16_t* y1, bf16_t* y2, bf16_t* y3,
                        hipStream_t stream) {
  const dim3 grid((unsigned)(N / kSmallRows));
  if (T <= 16)
    hipLaunchKernelGGL((proj_small_kernel<kFused, 1>), grid, dim3(256), 0, stream, x, T, K, w,
                       w_gate, N, y0, y1, y2, y3);
  else
    hipLaunchKernelGGL((proj_small_kernel<kFused, 2>), grid, dim3(256), 0, stream, x, T, K, w,
                       w_gate, N, y0, y1, y2, y3);
  return hipGetLastError();
}

// Workgroups for nN x nT tiles: with the XCD banding, 8 bands of ceil(nT / 8) token tiles.
long long grid_size(int nN, int nT) {
  return nT >= 8 ? 8LL * nN * ((nT + 7) / 8) : (long long)nN * nT;
}

}  // namespace

hipError_t launch_qkv_proj(const bf16_t* x, int T, const bf16_t* w_qkv, const bf16_t* w_gate,
                           bf16_t* q, bf16_t* k, bf16_t* v, bf16_t* gate, hipStream_t stream) {
  const int N = kQkvDim + kGateRows;
  if (T <= kSmallMaxT)
    return launch_small<1>(x, T, kProjHidden, w_qkv, w_gate, N, q, k, v, gate, stream);
  const int nN = (N + kTile - 1) / kTile, nT = (T + kTile - 1) / kTile;
  hipLaunchKernelGGL(proj_kernel<1>, dim3((unsigned)grid_size(nN, nT)), dim3(256), 0, stream, x, T,
                     kProjHidden, w_qkv, w_gate, N, q, k, v, gate, nN, nT);
  return hipGetLastError();
}

hipError_t launch_o_proj(const bf16_t* a, int T, const bf16_t* w_o, bf16_t* y,
                         hipStream_t stream) {
  if (T <= kSmallMaxT)
    return launch_small<0>(a, T, kQDim, w_o, nullptr, kProjHidden, y, nullptr, nullptr, nullptr,
                           stream);
  const int nN = kProjHidden / kTile, nT = (T + kTile - 1) / kTile;
  hipLaunchKernelGGL(proj_kernel<0>, dim3((unsigned)grid_size(nN, nT)), dim3(256), 0, stream, a, T,
                     kQDim, w_o, nullptr, kProjHidden, y, nullptr, nullptr, nullptr, nN, nT);
  return hipGetLastError();
}

}  // namespace hattn
