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
// Design (one workgroup = one KV head x 32 or 64 query positions, 4 or 8 waves):
//   * wave w owns query head 4*kvh + w%4 and one 32-row block, so every K/V tile staged in
//     LDS feeds all 4 heads of its group (and both row blocks when 8 waves share it);
//   * S^T = K . Q^T and O^T = V^T . P^T run on v_mfma_f32_32x32x16_bf16 with fp32
//     accumulation; a lane holds one query row's scores, so the online-softmax max needs
//     one cross-lane exchange (lane ^ 32) and the rescale of O is lane-local;
//   * 32-key K and V tiles go global -> LDS directly (the buffer form of the LDS copy, no
//     staging registers), row-major with an XOR swizzle of the 16-byte blocks; K tiles
//     rotate through two LDS stages and V tiles through three; the V^T operand is read
//     with ds_read_b64_tr_b16, which transposes 4 keys x 16 dims per lane group, in the key
//     order in which a lane already holds P^T in its accumulator;
//   * the loop is rotated: iteration t runs the PV step of tile t - 1 first (its
//     probabilities wait in registers), then issues the copies of tile t + 1, then QK and
//     the softmax of tile t.  The compiler drains every pending LDS copy before a
//     transposing read, so those reads are placed right after the barrier that waits for
//     the copies anyway, and the issue of the next copies overlaps PV MFMAs in flight;
//   * the row max used for exp2 only moves when a tile beats it by more than 2^8, so O is
//     rescaled rarely (probabilities stay <= 256 in between, exact in fp32 and bf16 range);
//   * tiles wholly outside the causal / sliding band are never visited (per workgroup, and
//     per wave for the row blocks of an 8-wave group); only tiles that straddle the band
//     edge, the diagonal or the cache end evaluate the element mask;
//   * optional fused Q-RoPE: the workgroup computes cos/sin of its positions once into
//     LDS and each lane rotates its own Q fragment (pairs d, d + r/2 sit in the same lane);
//   * epilogue: 1/l, sigmoid gate, bf16 store, optional fp32 LSE.
//
// Ring mode (sliding layers only): a chunk at positions pos0.. continues a 512-slot ring
// (slot = position mod 512).  Key positions stay absolute and tiles stay 32-aligned, so a
// tile below pos0 is one contiguous run of ring slots, a tile at or past pos0 is a run of
// the chunk's own rows, and only the tile that holds pos0 mixes the two, lane by lane.
// [T2] "The real bottleneck of a million-token context" (sliding layers keep only the
// most recent 512 tokens' keys and values).
#include "hattn_device.h"
#include "hattn_launch.h"

namespace hattn {

namespace {

constexpr int kBN = 32;                  // keys per tile
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleLog2 = 8.f;      // move the running max only when beaten by 2^8
constexpr int kRingSlots = 512;          // sliding-layer ring: one slot per window position

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// LDS tile row (one key, 512 bytes): 16-byte block b sits at block b ^ swz(r), a
// permutation of 0..7 over r & 7.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

// The value of lane l ^ 32 alongside lane l's own: v_permlane32_swap exchanges the two
// half-waves of a register pair in one VALU op (no LDS round trip).  Returns {x_l, x_(l^32)}
// in some order, which is all that a max or a sum needs.
__device__ __forceinline__ void halves(float x, float* a, float* b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  *a = __uint_as_float(r[0]);
  *b = __uint_as_float(r[1]);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Buffer resource for the copies of one tile (raw addressing, no stride; every offset a
// copy uses is below 2^31, so the range check never clips).  The buffer form of the
// global->LDS copy is counted on the vector-memory counter only, so the LDS reads that
// follow it keep exact lgkmcnt waits.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff,
                                           0x00020000);
}

// This wave's share of a 32-row tile load straight into LDS.  The tile is 16 KiB = 16
// wave-instructions of 1 KiB; wave w issues instructions w*nw .. w*nw + nw - 1.
// Instruction j fills LDS bytes [j*1024, +1024): lane l's 16 bytes land at position
// p = j*64 + l, i.e. row p/32, physical block p%32, so it fetches the logical block the
// swizzle maps there.  The per-lane source offsets (bytes from the tile's first row) do not
// depend on the tile, so they are computed once; the tile base is wave-uniform.
template <int kWaves>
struct TileLoader {
  static constexpr int nw = 16 / kWaves;
  static constexpr int kRowBytes = kHkv * kD * 2;  // cache row stride (4 KV heads)
  int lrow[nw];   // tile row each load instruction of this lane reads
  int lblk[nw];   // logical 16-byte block within that row

  __device__ __forceinline__ TileLoader(int w, int lane) {
#pragma unroll
    for (int i = 0; i < nw; ++i) {
      const int p = (nw * w + i) * 64 + lane;
      lrow[i] = p >> 5;
      lblk[i] = (p & 31) ^ swz(p >> 5);
    }
  }

  // Tile rows row0 .. row0 + 31 of `base`.  Rows past `last` (the last row any query of
  // the workgroup can see) read row `last` instead: their scores are masked to -inf, and
  // this way no row that the caller may not have written yet is ever read.
  __device__ __forceinline__ void load(char* dst, const bf16_t* base, int row0, int last,
                                       int w) const {
    const char* tile = reinterpret_cast<const char*>(base) + (long long)row0 * kRowBytes;
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(tile);
    const bool tail = row0 + kBN - 1 > last;
#pragma unroll
    for (int i = 0; i < nw; ++i) {
      const int r = tail ? min(lrow[i], last - row0) : lrow[i];
      const unsigned off = (unsigned)r * kRowBytes + (unsigned)lblk[i] * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + (nw * w + i) * 1024), 16,
                                               (int)off, 0, 0, 0);
    }
  }

  // Ring mode, the one tile holding the chunk start: key positions key0 .. key0 + 31,
  // those below pb from ring slot (position mod 512), the others from chunk row
  // position - pb (at most 31, clamped to last_row).  Each lane issues the copy from its own
  // source under a partial exec mask, so the tile can take up to twice the usual number
  // of copy instructions; the caller then waits for all of them.
  __device__ __forceinline__ void load_split(char* dst, const bf16_t* ring, const bf16_t* chunk,
                                             int key0, int pb, int last_row, int w) const {
    const __amdgpu_buffer_rsrc_t rr = tile_rsrc(ring);
    const __amdgpu_buffer_rsrc_t rc = tile_rsrc(chunk);
#pragma unroll
    for (int i = 0; i < nw; ++i) {
      const int j = key0 + lrow[i];
      lds_void* d = (lds_void*)(dst + (nw * w + i) * 1024);
      if (j < pb) {
        const unsigned off = (unsigned)(j & (kRingSlots - 1)) * kRowBytes + (unsigned)lblk[i] * 16u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, d, 16, (int)off, 0, 0, 0);
      } else {
        const unsigned off = (unsigned)min(j - pb, last_row) * kRowBytes + (unsigned)lblk[i] * 16u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, d, 16, (int)off, 0, 0, 0);
      }
    }
  }
};

// Wait until at most n of this wave's global->LDS copies are still in flight.
template <int n>
__device__ __forceinline__ void wait_lds_dma() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
}

// kc / vc: the position-indexed caches [B, cap, 4, 256], or in ring mode the chunk's own
// keys / values [B, Sq, 4, 256] with the rings kr / vr [B, 512, 4, 256].
template <bool kSliding, int kWaves, bool kRing>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc,
                    const bf16_t* __restrict__ vc, const bf16_t* __restrict__ kr,
                    const bf16_t* __restrict__ vr, int cap, const int* __restrict__ pos0, int B,
                    int Sq, const bf16_t* __restrict__ gate, bf16_t* __restrict__ out,
                    float* __restrict__ lse, int window, int rope_q, RopeTable tab, float sl2,
                    int nqb, int nwork) {
  static_assert(kSliding || !kRing, "ring mode is for sliding layers");
  constexpr int kThreads = 64 * kWaves;
  constexpr int kRB = kWaves / kGroup;       // 32-row blocks per workgroup
  constexpr int kBQ = 32 * kRB;              // query positions per workgroup
  constexpr int kHalf = kSliding ? 128 : 32;  // rot_dim / 2
  constexpr int kNdc = kHalf / 16;           // Q fragments holding the first rotary half
  constexpr int kTile = kBN * kD * 2;        // bytes of one K or V tile
  constexpr int kPitch = kHalf + 2;          // cos/sin table row, f32x2; +16 B vs bank aliasing
  constexpr int kCsBytes = kBQ * kPitch * 8;
  // 32-key tiles per barrier: 2 on full layers (their one workgroup per CU can take all
  // 160 KiB of LDS), 1 on sliding layers (two workgroups per CU share it).
  constexpr int kTPI = kSliding ? 1 : 2;
  constexpr int kRingBytes = 5 * kTPI * kTile;  // K tiles: 2 stages, V tiles: 3, of kTPI each
  constexpr int kLdsBytes = kRingBytes > kCsBytes ? kRingBytes : kCsBytes;
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int rb = w / kGroup;                 // this wave's row block

  int qb, b, kvh;
  if (kSliding) {
    // Equal work per workgroup: each XCD (blockIdx % 8) gets a contiguous run of query
    // blocks, so the K/V tiles that neighbouring blocks share stay in that XCD's L2.
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
  const int h = kvh * kGroup + (w % kGroup);
  const int i0 = qb * kBQ;
  const int nrows = min(kBQ, Sq - i0);
  // Clamped so that positions up to pb + Sq - 1 cannot overflow.
  const int pb = min(pos0[b], 0x7fffffff - Sq);
  const int P0 = pb + i0;
  const int Plast = P0 + nrows - 1;
  // This wave's rows: 32rb .. 32rb + 31 of the workgroup.
  const int r0 = 32 * rb;
  const bool row_ok = r0 + n < nrows;
  const int row_i = i0 + (row_ok ? r0 + n : 0);
  const int prow = P0 + r0 + n;
  const int Pw0 = P0 + r0;                           // first row position of this wave
  const int Pwl = P0 + min(r0 + 31, nrows - 1);      // last valid row position of this wave

  // In ring mode every visible key exists (older ones in the ring, newer in the chunk).
  const int capk = kRing ? Plast + 1 : cap;
  const long long kv_off = ((long long)b * (kRing ? Sq : cap) * kHkv + kvh) * kD;
  const bf16_t* kbase = kc + kv_off;
  const bf16_t* vbase = vc + kv_off;
  const long long ring_off = kRing ? ((long long)b * kRingSlots * kHkv + kvh) * kD : 0;
  const bf16_t* krbase = kr + ring_off;
  const bf16_t* vrbase = vr + ring_off;
  const int kmax = min(Plast, capk - 1);
  const int kmin = kSliding ? max(0, P0 - (window - 1)) : 0;
  const bool any_keys = kmax >= kmin;
  const int t_lo = any_keys ? kmin / kBN : 0;
  const int t_hi = any_keys ? kmax / kBN : -1;
  // Tiles this wave's rows can see at all (a workgroup's row blocks see different bands).
  const int wt_lo = kSliding ? max(0, Pw0 - (window - 1)) / kBN : 0;
  const int wt_hi = min(Pwl, capk - 1) / kBN;

  // The cos/sin table's column is tid mod kHalf on every pass, so each thread needs one
  // frequency.  It is read before the Q rows: loads complete in issue order, and behind
  // them its wait would also wait for all of Q.
  static_assert(kThreads % kHalf == 0, "a thread keeps one table column");
  const int fcol = tid & (kHalf - 1);
  const float freq = rope_q ? tab.inv_freq[fcol] : 0.f;

  // Q^T operand: lane (n, hh) holds dims 16dc + 8hh .. +7 of query row n of this wave.
  bf16x8 qf[16];
  {
    const bf16_t* qrow = q + (((long long)b * Sq + row_i) * kHq + h) * kD + 8 * hh;
#pragma unroll
    for (int dc = 0; dc < 16; ++dc) {
      qf[dc] = row_ok ? *reinterpret_cast<const bf16x8*>(qrow + 16 * dc) : bf16x8{};
    }
  }

  if (rope_q) {
    f32x2* cs = reinterpret_cast<f32x2*>(smem);
    for (int r = tid / kHalf; r < kBQ; r += kThreads / kHalf) {
      float sv, cv;
      sincos_angle(rope_angle(P0 + r, freq), &sv, &cv);
      cs[r * kPitch + fcol] = f32x2{cv, sv};
    }
    __syncthreads();
#pragma unroll
    for (int dc = 0; dc < kNdc; ++dc) {
      const f32x2* c8 = cs + (r0 + n) * kPitch + 16 * dc + 8 * hh;
      rope_fragments(qf[dc], qf[dc + kNdc], [&](int e) { return c8[e]; });
    }
    __syncthreads();  // the cos/sin table shares LDS with the first tiles
  }

  // Per-lane LDS address parts that do not depend on the tile.
  const int ksw = swz(n);  // K operand: row n, block 2dc + hh
  // V^T operand via ds_read_b64_tr_b16: within 16-lane group g = lane/16, lane i supplies
  // the 8 bytes at key 4hh + i/4 (+16c, +8 for the second half), dims 16(g&1) + 4(i&3)
  // (+32mb); the instruction hands lane i the 4 keys of dim 16(g&1) + i.
  const int gi = lane & 15;
  const int trow = 4 * hh + (gi >> 2);
  const int tdim = 16 * ((lane >> 4) & 1) + 4 * (gi & 3);
  const int tsw = swz(trow);
  const int tlo = (tdim & 7) * 2;  // 0 or 8 bytes into the 16-byte block

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) o[mb] = f32x16{};
  const TileLoader<kWaves> ld(w, lane);
  // K and V tile t (key positions 32t .. 32t + 31) into LDS at kd and vd.
  auto load_tile = [&](char* kd, char* vd, int t) {
    const int key0 = t * kBN;
    if (!kRing) {
      ld.load(kd, kbase, key0, kmax, w);
      ld.load(vd, vbase, key0, kmax, w);
    } else if (key0 >= pb || key0 + kBN <= pb) {
      // One source for the whole tile: a run of the chunk's rows, or of ring slots (tiles
      // are 32-aligned, so a ring run does not wrap).  A single load() call for both keeps
      // the per-lane offsets 32-bit and computed per tile.
      const bool in_ring = key0 < pb;
      const int row0 = in_ring ? (key0 & (kRingSlots - 1)) : key0 - pb;
      const int last = in_ring ? row0 + kBN - 1 : kmax - pb;
      ld.load(kd, in_ring ? krbase : kbase, row0, last, w);
      ld.load(vd, in_ring ? vrbase : vbase, row0, last, w);
    } else {
      ld.load_split(kd, krbase, kbase, key0, pb, kmax - pb, w);
      ld.load_split(vd, vrbase, vbase, key0, pb, kmax - pb, w);
    }
  };
  // Each wave raises its issue priority while it issues the PV MFMAs, the copies and the QK
  // chain, and drops it for the softmax, so that the other wave on its SIMD (on sliding
  // layers, of another workgroup) keeps the MFMA pipe busy meanwhile: 0.6-0.8% on the 32K
  // sliding prefill, 0.4% on the full 1M chunk.  (A static raised priority for row block 0
  // of the full layers, which staggered the softmax phases at one tile per barrier, was
  // 0.3-0.6% slower with two tiles per barrier.)
  if (kSliding) __builtin_amdgcn_s_setprio(2);

  // K tiles rotate through two LDS stages and V tiles through three, each stage holding
  // kTPI tiles.  An iteration takes the kTPI tiles from t: it first runs the PV steps of
  // the previous iteration's tiles (their probabilities wait in registers), then issues
  // the copies of the next kTPI tiles, then QK and the softmax of its own.  So the
  // transposing V reads follow a barrier that has already drained the copies, and the
  // issue of the next copies overlaps the PV MFMAs still in the pipe.  With two tiles per
  // barrier the softmax of the last wave to finish its QK, which nothing else on its SIMD
  // overlaps before the barrier, comes once per 64 keys instead of once per 32.
  char* const kring = smem;
  char* const vring = smem + 2 * kTPI * kTile;
  auto qk_softmax = [&](const char* kst, int t, bf16x8* pfo) __attribute__((always_inline)) {
    // S^T[key][query]; accumulator element 4i + j of lane half hh is key 8i + 4hh + j.
    // K fragments are read two ahead of the MFMA that consumes them.
    auto kfrag = [&](int dc) {
      const int blk = ((2 * dc + hh) & 7) ^ ksw;
      return *reinterpret_cast<const bf16x8*>(kst + n * 512 + (dc >> 2) * 128 + (blk << 4));
    };
    f32x16 s = f32x16{};
    bf16x8 ka = kfrag(0), kb = kfrag(1);
#pragma unroll
    for (int dc = 0; dc < 16; ++dc) {
      const bf16x8 kn = dc + 2 < 16 ? kfrag(dc + 2) : kb;
      s = mfma32(ka, qf[dc], s);
      ka = kb;
      kb = kn;
    }
    // Keep two LDS reads in flight ahead of the MFMA chain.
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < 14; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_s_setprio(0);

    const int key0 = t * kBN;
    const bool whole = (key0 <= Pw0 - (kBN - 1)) && (key0 <= capk - kBN) &&  // no key0 + kBN:
                       (!kSliding || Pwl - key0 <= window - 1);    // it overflows near 2^31
    if (!whole) {
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        const int j = key0 + 8 * (idx >> 2) + 4 * hh + (idx & 3);
        const bool vis = j <= prow && j < capk && (!kSliding || prow - j <= window - 1);
        s[idx] = vis ? s[idx] : -INFINITY;
      }
    }
    // Row max of the raw scores, then scaled (sl2 > 0 commutes with max).
    float mloc = -INFINITY;
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) mloc = fmaxf(mloc, s[idx]);
    {
      float a, b;
      halves(mloc, &a, &b);
      mloc = fmaxf(a, b) * sl2;
    }
    // Move the reference max only when the tile beats it by more than 2^8 (or on a row's
    // first visible key); otherwise probabilities stay below 256 and O is left alone.
    const bool bump = mloc > m_run + kRescaleLog2 || (m_run == -INFINITY && mloc != -INFINITY);
    if (__any(bump)) {
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) o[mb] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float rs = 0.f;
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) {
      const float p = fast_exp2(__builtin_fmaf(s[idx], sl2, -m_use));
      s[idx] = p;
      rs += p;
    }
    l_run += rs;

    // O^T += V^T P^T.  P^T of 16-key chunk c is accumulator elements 8c .. 8c+7.
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const f32x4 lo = {s[8 * c], s[8 * c + 1], s[8 * c + 2], s[8 * c + 3]};
      const f32x4 hi = {s[8 * c + 4], s[8 * c + 5], s[8 * c + 6], s[8 * c + 7]};
      const bf16x4 pl = __builtin_convertvector(lo, bf16x4);
      const bf16x4 ph = __builtin_convertvector(hi, bf16x4);
      pfo[c] = bf16x8{pl[0], pl[1], pl[2], pl[3], ph[0], ph[1], ph[2], ph[3]};
    }
  };
  auto pv = [&](const char* vst, const bf16x8* pfi) __attribute__((always_inline)) {
    // V^T fragment i = 8c + mb: keys 16c + trow (slots 0..3) and 16c + 8 + trow (slots
    // 4..7), dims 32mb + 16(g&1) + ..; read three MFMAs ahead of its use (measured: the
    // transposing reads need more cover than the K reads, which run two ahead).
    auto vfrag = [&](int i) {
      const int c = i >> 3, mb = i & 7;
      const int blk = ((4 * mb + (tdim >> 3)) & 7) ^ tsw;
      const int off = (16 * c + trow) * 512 + (mb >> 1) * 128 + (blk << 4) + tlo;
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vst + off));
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vst + off + 8 * 512));
      return __builtin_bit_cast(bf16x8,
                                s16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
    };
    constexpr int kVAhead = 3;
    bf16x8 vq[kVAhead];
#pragma unroll
    for (int a = 0; a < kVAhead; ++a) vq[a] = vfrag(a);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bf16x8 vn = i + kVAhead < 16 ? vfrag(i + kVAhead) : vq[0];
      o[i & 7] = mfma32(vq[0], pfi[i >> 3], o[i & 7]);
#pragma unroll
      for (int a = 0; a + 1 < kVAhead; ++a) vq[a] = vq[a + 1];
      vq[kVAhead - 1] = vn;
    }
    // Two transposing reads per fragment: 2 * kVAhead up front, then two per MFMA.
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kVAhead, 1);
#pragma unroll
    for (int i = 0; i < 16 - kVAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kVAhead, 1);
  };

  if constexpr (kTPI == 1) {
    if (t_lo <= t_hi) load_tile(kring, vring, t_lo);
    bf16x8 pf[2];
    bool have_p = false;
    int vcur = 0;  // V stage of tile t
    for (int t = t_lo; t <= t_hi; ++t) {
      const int it = t - t_lo;
      // Tile t has landed for every wave, and every wave is done with iteration t - 1.
      wait_lds_dma<0>();
      __syncthreads();
      const int vprev = vcur == 0 ? 2 : vcur - 1;
      const int vnext = vcur == 2 ? 0 : vcur + 1;
      if (kSliding) __builtin_amdgcn_s_setprio(2);
      if (have_p) pv(vring + vprev * kTile, pf);
      if (t + 1 <= t_hi) load_tile(kring + ((it + 1) & 1) * kTile, vring + vnext * kTile, t + 1);
      have_p = t >= wt_lo && t <= wt_hi;
      if (have_p) qk_softmax(kring + (it & 1) * kTile, t, pf);
      vcur = vnext;
    }
    if (have_p) pv(vring + (vcur == 0 ? 2 : vcur - 1) * kTile, pf);
  } else {
    // Two tiles per barrier: PV of the previous iteration's second tile, the copies of the
    // next two, then QK, softmax and PV of tile t, then QK and softmax of tile t + 1, whose
    // probabilities wait for the next iteration.  Only one tile's probabilities are live
    // across the barrier.
    //
    // Row block 0 runs that last PV before the barrier instead.  The two waves sharing a
    // SIMD are w and w + 4, one of each row block.  With the same order in both, the row
    // block 0 wave ran ahead and waited about 900 clocks per iteration at the barrier while
    // its partner finished QK and softmax alone, so the MFMA pipe idled during that softmax.
    // Moving one PV step across the barrier for one of the two offsets them, and each
    // softmax then meets the other wave's MFMAs: 2.6% on the 1M chunk, 3.1% at 128K.
    if (t_lo <= t_hi) load_tile(kring, vring, t_lo);
    if (t_lo + 1 <= t_hi) load_tile(kring + kTile, vring + kTile, t_lo + 1);
    bf16x8 pf[2];
    bool have_p = false;
    int vcur = 0;  // V stage of tiles t, t + 1
    for (int t = t_lo; t <= t_hi; t += 2) {
      const int kcur = ((t - t_lo) >> 1) & 1;  // their K stage
      // Tiles t and t + 1 have landed for every wave, and every wave is done with the
      // previous iteration.
      wait_lds_dma<0>();
      __syncthreads();
      const int vprev = vcur == 0 ? 2 : vcur - 1;
      const int vnext = vcur == 2 ? 0 : vcur + 1;
      __builtin_amdgcn_s_setprio(2);
      if (have_p) pv(vring + (2 * vprev + 1) * kTile, pf);
      if (t + 2 <= t_hi)
        load_tile(kring + (2 * (kcur ^ 1)) * kTile, vring + (2 * vnext) * kTile, t + 2);
      if (t + 3 <= t_hi)
        load_tile(kring + (2 * (kcur ^ 1) + 1) * kTile, vring + (2 * vnext + 1) * kTile, t + 3);
      if (t >= wt_lo && t <= wt_hi) {
        qk_softmax(kring + (2 * kcur) * kTile, t, pf);
        __builtin_amdgcn_s_setprio(2);
        pv(vring + (2 * vcur) * kTile, pf);
      }
      have_p = t + 1 <= t_hi && t + 1 >= wt_lo && t + 1 <= wt_hi;
      if (have_p) qk_softmax(kring + (2 * kcur + 1) * kTile, t + 1, pf);
      if (rb == 0) {
        if (have_p) {
          __builtin_amdgcn_s_setprio(2);
          pv(vring + (2 * vcur + 1) * kTile, pf);
        }
        have_p = false;
      }
      vcur = vnext;
    }
    if (have_p) pv(vring + (2 * (vcur == 0 ? 2 : vcur - 1) + 1) * kTile, pf);
  }

  float l_a, l_b;
  halves(l_run, &l_a, &l_b);
  const float l_tot = l_a + l_b;
  // row_i is a valid row in every lane (clamped above), so all lanes take part in the
  // exchange below; only rows that exist are stored.
  const long long row = (long long)b * Sq + row_i;
  const float g = bf16_to_f32(gate[row * kHq + h]);
  const float sg = 1.f / (1.f + expf(-g));
  const float f = l_tot > 0.f ? sg / l_tot : 0.f;
  // O^T accumulator element 4i + j of block mb is dim 32mb + 8i + 4hh + j: a lane holds
  // 4-dim pieces of its row.  v_permlane32_swap trades pieces between the lanes hh = 0 and
  // hh = 1 of one row (lanes n and n + 32): for each pair of pieces (i = 2ip, 2ip + 1) the
  // hh = 1 lane hands over its piece 2ip and the hh = 0 lane its piece 2ip + 1, so lane
  // hh = 0 ends with dims 16ip + 0..7 and lane hh = 1 with dims 16ip + 8..15 of the block,
  // 16 contiguous bytes each.
  uint4 ov[8][2];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
    for (int ip = 0; ip < 2; ++ip) {
      const int e = 8 * ip;  // piece 2ip starts at accumulator element 8ip
      const uint32_t a0 = pack_bf16x2(o[mb][e] * f, o[mb][e + 1] * f);
      const uint32_t a1 = pack_bf16x2(o[mb][e + 2] * f, o[mb][e + 3] * f);
      const uint32_t c0 = pack_bf16x2(o[mb][e + 4] * f, o[mb][e + 5] * f);
      const uint32_t c1 = pack_bf16x2(o[mb][e + 6] * f, o[mb][e + 7] * f);
      // Upper lanes of the first operand trade with lower lanes of the second.
      const auto s0 = __builtin_amdgcn_permlane32_swap(a0, c0, false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(a1, c1, false, false);
      ov[mb][ip] = uint4{s0[0], s1[0], s0[1], s1[1]};
    }
  }
  if (row_ok) {
    bf16_t* orow = out + (row * kHq + h) * kD + 8 * hh;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
      for (int ip = 0; ip < 2; ++ip) {
        *reinterpret_cast<uint4*>(orow + 32 * mb + 16 * ip) = ov[mb][ip];
      }
    }
    if (lse != nullptr && hh == 0) {
      lse[row * kHq + h] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

// Launch shapes, measured on MI355X: full-causal rows stream long K/V prefixes, so 8 waves
// (two 32-row blocks per head) share each staged tile and halve L2 requests; sliding rows
// see a 512-key band, where 32-row blocks waste fewer keys at the band edges.
constexpr int kWavesFull = 8;
constexpr int kWavesSliding = 4;

template <bool kSliding, int kWaves, bool kRing>
hipError_t launch_kind(const bf16_t* q, const bf16_t* k_cache, const bf16_t* v_cache,
                       const bf16_t* k_ring, const bf16_t* v_ring, int cap, const int* pos0,
                       int B, int Sq, const bf16_t* gate, bf16_t* out, float* lse, int window,
                       bool rope_q, const RopeTable& tab, float scale_log2e, hipStream_t stream) {
  constexpr int kBQ = 32 * (kWaves / kGroup);
  const int nqb = (Sq + kBQ - 1) / kBQ;
  const long long nwork = (long long)B * kHkv * nqb;
  // Sliding grids are padded to a multiple of 8 for the XCD-contiguous mapping.
  const long long grid = kSliding ? (nwork + 7) / 8 * 8 : nwork;
  hipLaunchKernelGGL((prefill_kernel<kSliding, kWaves, kRing>), dim3((unsigned)grid),
                     dim3(64 * kWaves), 0, stream, q, k_cache, v_cache, k_ring, v_ring, cap, pos0,
                     B, Sq, gate, out, lse, window, rope_q ? 1 : 0, tab, scale_log2e, nqb,
                     (int)nwork);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const bf16_t* q, const bf16_t* k_cache, const bf16_t* v_cache, int cap,
                          const int* pos0, int B, int Sq, const bf16_t* gate, bf16_t* out,
                          float* lse, int window, bool rope_q, const RopeTable& tab,
                          float scale_log2e, hipStream_t stream) {
  if (window > 0)
    return launch_kind<true, kWavesSliding, false>(q, k_cache, v_cache, nullptr, nullptr, cap,
                                                   pos0, B, Sq, gate, out, lse, window, rope_q,
                                                   tab, scale_log2e, stream);
  return launch_kind<false, kWavesFull, false>(q, k_cache, v_cache, nullptr, nullptr, cap, pos0, B,
                                               Sq, gate, out, lse, window, rope_q, tab,
                                               scale_log2e, stream);
}

hipError_t launch_prefill_ring(const bf16_t* q, const bf16_t* k_new, const bf16_t* v_new,
                               const bf16_t* k_ring, const bf16_t* v_ring, const int* pos0, int B,
                               int Sq, const bf16_t* gate, bf16_t* out, float* lse, int window,
                               bool rope_q, const RopeTable& tab, float scale_log2e,
                               hipStream_t stream) {
  if (window != kRingSlots) return hipErrorInvalidValue;
  return launch_kind<true, kWavesSliding, true>(q, k_new, v_new, k_ring, v_ring, Sq, pos0, B, Sq,
                                                gate, out, lse, window, rope_q, tab, scale_log2e,
                                                stream);
}

}  // namespace hattn
