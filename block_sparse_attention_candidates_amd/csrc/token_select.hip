// Token-level dynamic-threshold selection on gfx950 ([DR] §3.2
// "Dynamic-threshold mode", Eqs. 9-11, "Global thresholding with safeguards",
// Algorithm 1; aggregation by "Density control within blocks", §3.1).
// [DR] = "DynamicRad: Content-Adaptive Sparse Attention for Long Video
// Diffusion", arXiv 2604.20470.
//
// One mask per batch element, shared by every head. Launches:
//   stats:    a workgroup of 8 wavefronts owns 256 query tokens (8 / 4 query
//             blocks); it walks the union of their candidate key blocks in
//             ascending order, staging each key block of the H_f fused heads in
//             an LDS ring (XOR-swizzled rows) filled by 4 loader wavefronts
//             (see ring_load), and every compute wave whose
//             query block has the key block as a candidate computes its 32x32
//             token tiles of s = (1/H_f) sum_h Q^h K^h^T / sqrt(d_k) (Eq. 9) with
//             v_mfma_f32_32x32x16_bf16. Token pairs of P(i, j) with t > 1 feed
//             per-frame-pair statistics (count, mean, M2 merged with Chan's
//             formula in float64, and the highest score with its position);
//             each wave keeps its own LDS accumulators, merged in a fixed order
//             into one partial per workgroup: no floating-point atomics.
//             At B_s <= 64 it also stores, for 32 x 32 tiles whose query rows
//             lie in one frame, each key column's float32 sum and sum of
//             squares of its logits in P.
//   reduce:   per frame pair, the workgroup partials merged in workgroup order:
//             mu, sigma (population), tau(t) by decay state (Eq. 11), and the
//             threshold in score units thr = mu + tau * (sigma + eps) (Eq. 10
//             rearranged), rounded up to float so that s >= thr in float32 is
//             exactly (double) s >= mu + tau * (sigma + eps). A frame pair is
//             served iff its highest score reaches thr.
//   mark:     a pair is selected iff it is a candidate pair (Eqs. 6-7) and
//             t <= 1 (tau = -inf) or s >= thr. Per block pair, key tokens are
//             active iff their selected share of the query tokens exceeds
//             theta_c, and the block pair is kept iff the active share of the
//             key tokens exceeds theta_m; one flag per candidate entry.
//             B_s = 128: the stats pass's walk and tiles (mark_kernel).
//             B_s <= 64: decide_kernel fixes every flag that the column sums
//             determine (exact counts, or Cantelli bounds on each column's
//             count), and mark_open_kernel computes the tiles of the rest.
//   fallback: for each unserved frame pair (safeguard (ii)), the block pair
//             holding its highest-scoring pair is re-decided with that pair
//             added, by the same tile and selection code.
//   compact:  one wavefront per (b, query block): flags -> ascending kept list,
//             written for every head (flag_compact_kernel, shared with the
//             static decay-state selector).
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "dr_internal.h"
#include "token.h"
#include "lds_dma.h"

namespace dr {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 8;              // compute wavefronts
constexpr int kLoadWaves = 4;          // loader wavefronts (key-block copies only)
constexpr int kThreads = (kWaves + kLoadWaves) * 64;
constexpr int kRows = kWaves * 32;      // query tokens per workgroup
constexpr int kRingMax = 16;            // ring depth limit (key blocks)
constexpr int kTokLdsBytes = 160 * 1024; // LDS per workgroup on gfx950
constexpr int kDone = 0x3fffffff;       // progress of a wave that reads no more blocks
constexpr int kOpenChunk = 16;          // candidate entries per wavefront of mark_open_kernel
constexpr int kDecideUnroll = 4;        // entries per lane group of decide_kernel with loads in flight
// Block sizes whose mark pass is the decision pass plus the open-entry kernel
// (one block pair = (B_s / 32)^2 tiles of 32 x 32, each with its own column sums).
constexpr int kDecideMaxBs = 64;

typedef int intx4 __attribute__((ext_vector_type(4)));
#define DR_LDS __attribute__((address_space(3)))

// Set (kWaitToken) by a wave whose bounded ring wait gave up; read and cleared
// by the host (take_wait_flags_token).
__device__ unsigned int g_tok_wait_flags;
__device__ __forceinline__ int ld_relaxed(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void st_relaxed(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Sum of a value over lanes l and l ^ 32, the same float in both:
// v_permlane32_swap(v, v) gives the low half's value in one result and the
// high half's in the other.
__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// order-preserving unsigned key of a float
__device__ __forceinline__ unsigned int fkey(float s) {
  unsigned int u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned long long pack_max(float s, unsigned int loc) {
  return ((unsigned long long)fkey(s) << 32) | (unsigned long long)(0xffffffffu - loc);
}

// XOR swizzle of 16-byte chunks within a staged key row (same layout argument
// as the attention kernel: 16 lanes read 16 rows at one logical chunk)
template <int D>
__device__ __forceinline__ int swz(int key) { return D == 128 ? (key & 15) : ((key >> 1) & 7); }

using Stat = TokStat;

// Chan et al.'s pairwise update: merge (nb, mb, m2b) into a.
__device__ __forceinline__ void merge(Stat& a, double nb, double mb, double m2b, unsigned long long mxb) {
  if (mxb > a.mx) a.mx = mxb;
  if (nb == 0.0) return;
  if (a.n == 0.0) {
    a.n = nb;
    a.mean = mb;
    a.m2 = m2b;
    return;
  }
  const double n = a.n + nb;
  const double d = mb - a.mean;
  a.mean += d * (nb / n);
  a.m2 += m2b + d * d * (a.n * nb / n);
  a.n = n;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ unsigned long long wave_max(unsigned long long v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const unsigned long long o = __shfl_xor(v, off);
    v = o > v ? o : v;
  }
  return v;
}

template <int D, int BS, int HF>
struct Geo {
  static constexpr int RB = 2 * D;                  // bytes per staged key row
  static constexpr int KBUF = HF * BS * RB;         // one key block, all fused heads
  static constexpr int QB = kRows / BS;             // query blocks per workgroup
  static constexpr int WPQ = BS / 32;               // waves per query block
  static constexpr int NI = KBUF / 1024;            // 1 KB direct-to-LDS loads per block
};

// Fused-head logits of one 32x32 token tile: A = this wave's Q rows (registers),
// B = 32 staged keys (key sub-block ksub of the staged block). Lane l gets key
// column l%32 and query rows 8*(i/4) + 4*(l/32) + i%4. The key operands are
// read two products ahead, in an order the scheduler may not change: left to
// itself, under the register limit of three waves per SIMD, it waits for each
// read right before its product (wan14b_720p + "mid" 4.84 -> 4.73 ms per
// selection; three ahead spill more and gain nothing).
template <int D, int BS, int HF>
__device__ __forceinline__ floatx16 tile_scores(const bf16x8 (&qf)[HF][D / 16], const unsigned char* kbuf, int ksub,
                                       int lane) {
  using G = Geo<D, BS, HF>;
  constexpr int NK = HF * (D / 16);      // products per tile
  constexpr int PF = 2;                  // key operands in flight
  floatx16 acc = {};
  const int key = 32 * ksub + (lane & 31), half = lane >> 5;
  auto operand = [&](int i) -> bf16x8 {
    const int h = i / (D / 16), kk = i - h * (D / 16);
    const unsigned char* row = kbuf + (h * BS + key) * G::RB;
    const int ch = (2 * kk + half) ^ swz<D>(key);
    return *reinterpret_cast<const bf16x8*>(row + ch * 16);
  };
  bf16x8 kb[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) kb[i] = operand(i);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int h = i / (D / 16), kk = i - h * (D / 16);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[h][kk], kb[i % PF], acc, 0, 0, 0);
    if (i + PF < NK) kb[i % PF] = operand(i + PF);
    __builtin_amdgcn_sched_barrier(0);
  }
  return acc;
}

// The Q fragments of 32 query rows starting at token q0 (rows >= S are zero).
template <int D, int HF>
__device__ __forceinline__ void load_q(const TokParams& p, int b, int q0, int lane, bf16x8 (&qf)[HF][D / 16]) {
  const int r = q0 + (lane & 31), half = lane >> 5;
#pragma unroll
  for (int h = 0; h < HF; ++h) {
    const uint16_t* src = p.q + ((size_t)(b * p.H + h) * p.S + (size_t)(r < p.S ? r : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 w = {0, 0, 0, 0};
      if (r < p.S) w = *reinterpret_cast<const u32x4*>(src + 16 * kk + 8 * half);
      qf[h][kk] = __builtin_bit_cast(bf16x8, w);
    }
  }
}

// Stage key block kb of batch b (all fused heads) into LDS buffer buf with
// direct-to-LDS loads issued by one wave: load n (64 lanes x 16 B) fills bytes
// [1024 n, 1024 n + 1024) of the buffer, that is chunk slots 64 n .. 64 n + 63
// in row-major order. Slot s of key row r holds the row's logical chunk
// s ^ swz(key), so the source address carries the swizzle. Keys >= S read the
// last token instead (finite values that no selection uses: tiles holding them
// take the masked path).
template <int D, int BS, int HF>
__device__ __forceinline__ void issue_block(const TokParams& p, int b, int kb, unsigned char* buf, int lane) {
  using G = Geo<D, BS, HF>;
#pragma unroll 4
  for (int n = 0; n < G::NI; ++n) {
    const int c = n * 64 + lane;
    const int row = c / (D / 8), slot = c % (D / 8);
    const int h = row / BS, key = row % BS;
    const int tok = min(kb * BS + key, p.S - 1);
    dma16(p.k + ((size_t)(b * p.H + h) * p.S + tok) * D + (size_t)(slot ^ swz<D>(key)) * 8, buf + n * 1024);
  }
}

// Per-lane view of one tile's token pairs: the lane's key token and, for its
// 16 query rows, which of the (at most two) query frames each row lies in.
struct TileFrames {
  int f0;        // frame of the wave's first query row
  int u0;        // its spatial index
  int fk, uk;    // this lane's key token frame and spatial index
  bool kvalid;
};

__device__ __forceinline__ TileFrames tile_frames(const TokParams& p, int q0, int ktok) {
  TileFrames f;
  f.f0 = q0 / p.Nt;
  f.u0 = q0 - f.f0 * p.Nt;
  f.kvalid = ktok < p.S;
  f.fk = ktok / p.Nt;
  f.uk = ktok - f.fk * p.Nt;
  return f;
}

// Frame and spatial index of a token given those of an earlier token of the
// same or an earlier frame, `add` tokens before it (no division).
struct FrameAt {
  int f, u;
};
__device__ __forceinline__ FrameAt frame_after(FrameAt at, int add, int Nt) {
  at.u += add;
  while (at.u >= Nt) {
    at.u -= Nt;
    ++at.f;
  }
  return at;
}

// The same view from the frames of the tile's first query and key tokens
// (lane key = k0 + lane % 32, N_t >= 32 so at most one frame boundary).
__device__ __forceinline__ TileFrames tile_frames_at(const TokParams& p, FrameAt q, FrameAt k, int k0, int lane) {
  TileFrames f;
  f.f0 = q.f;
  f.u0 = q.u;
  f.kvalid = k0 + (lane & 31) < p.S;
  const FrameAt kl = frame_after(k, lane & 31, p.Nt);
  f.fk = kl.f;
  f.uk = kl.u;
  return f;
}

// Row i of the lane: query token q0 + r, r = 8*(i/4) + 4*half + i%4.
__device__ __forceinline__ int row_of(int i, int half) { return 8 * (i >> 2) + 4 * half + (i & 3); }

// A 32x32 tile (query tokens q0.., key tokens k0..) lying inside one query
// frame and one key frame, away from the sequence end, has one frame distance
// t for all its pairs; then its pairs are all or none in P(i, j) unless the
// window edge cuts it. Computed in scalar registers.
enum TileClass { kGeneral = 0, kNone = 1, kAllNear = 2, kAllScored = 3, kCutNear = 4, kCutScored = 5 };
struct TileInfo {
  int cls, fq, fk;
};
__device__ __forceinline__ TileInfo classify(const TokParams& p, int q0, FrameAt q, int k0, FrameAt k, const int* s_w,
                                             const int* s_ret) {
  TileInfo ti{kGeneral, 0, 0};
  if (q0 + 31 >= p.S || k0 + 31 >= p.S) return ti;
  if (q.u + 31 >= p.Nt || k.u + 31 >= p.Nt) return ti;   // the tile crosses a frame boundary
  const int fq = q.f, fk = k.f;
  ti.fq = fq;
  ti.fk = fk;
  const int t = fq > fk ? fq - fk : fk - fq;
  if (!s_ret[t]) {
    ti.cls = kNone;
    return ti;
  }
  const int uq = q.u, uk = k.u, w = s_w[t];
  const int dmax = max(uq + 31 - uk, uk + 31 - uq);                  // largest |u - v| in the tile
  const int dmin = max(0, max(uk - (uq + 31), uq - (uk + 31)));      // smallest
  if (dmin > w) ti.cls = kNone;
  else if (dmax <= w) ti.cls = t <= 1 ? kAllNear : kAllScored;
  else ti.cls = t <= 1 ? kCutNear : kCutScored;   // the window edge cuts the tile
  return ti;
}

// A general tile whose 32 query rows lie in one frame, away from the sequence
// end: only its keys cross a frame boundary, so each key column lies in one
// frame pair.
__device__ __forceinline__ bool key_straddle(const TokParams& p, int q0, FrameAt q, int k0, const TileInfo& ti) {
  return ti.cls == kGeneral && q0 + 31 < p.S && k0 + 31 < p.S && q.u + 31 < p.Nt;
}

// Key-column sums of tile (row tile sub, key sub-block ksub) of candidate entry
// ent of batch element b: 32 (sum, sum of squares) pairs.
template <int BS>
__device__ __forceinline__ floatx2* colsum_of(const TokParams& p, int b, long long ent, int sub, int ksub) {
  constexpr int QS = BS / 32;
  return reinterpret_cast<floatx2*>(p.colsum) + (((size_t)b * p.nnz + (size_t)ent) * (QS * QS) + sub * QS + ksub) * 32;
}

// Selection bits (one per element i) of a tile under the thresholds of the
// frame pairs involved; inP bits mark the candidate pairs of P with t > 1.
// thr0 / thr1: thresholds (score units) for query frame f0 / f0 + 1 against
// the lane's key frame. s_w / s_ret: per-distance window and "retained"
// (t mod sf(t) = 0) tables in LDS.
__device__ __forceinline__ void select_bits(const TokParams& p, const floatx16& acc, const TileFrames& f, int q0, int half,
                                   const int* s_w, const int* s_ret, float thr0, float thr1, unsigned& sel,
                                   unsigned& inP2) {
  sel = 0;
  inP2 = 0;
  if (!f.kvalid) return;
  const int t0 = f.f0 > f.fk ? f.f0 - f.fk : f.fk - f.f0;
  const int t1 = f.f0 + 1 > f.fk ? f.f0 + 1 - f.fk : f.fk - f.f0 - 1;
  const bool ret0 = t0 < p.Nf && s_ret[t0];
  const bool ret1 = t1 < p.Nf && s_ret[t1];
  const int w0 = t0 < p.Nf ? s_w[t0] : 0, w1 = t1 < p.Nf ? s_w[t1] : 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = row_of(i, half);
    if (q0 + r >= p.S) continue;
    int u = f.u0 + r;
    const bool second = u >= p.Nt;
    if (second) u -= p.Nt;
    const int t = second ? t1 : t0;
    const bool ret = second ? ret1 : ret0;
    const int w = second ? w1 : w0;
    const int du = u > f.uk ? u - f.uk : f.uk - u;
    if (!ret || du > w) continue;
    if (t <= 1) {
      sel |= 1u << i;
    } else {
      inP2 |= 1u << i;
      if (acc[i] * p.scale >= (second ? thr1 : thr0)) sel |= 1u << i;
    }
  }
}

// LDS layout shared by the stats and mark kernels: the key-block ring (nb
// buffers, chosen at launch), per-query-block candidate bitmaps and their CSR word prefixes, the union
// bitmap, and the per-distance table; then kernel-specific areas.
constexpr int kCtlBytes = 128;   // ring control: prog[8], ready[16], padding

template <int D, int BS, int HF>
struct Lds {
  using G = Geo<D, BS, HF>;
  int nword;
  int nb;               // ring buffers (chosen at launch: the deepest ring that fits)
  unsigned char* ring;  // [nb][KBUF]
  unsigned int* bits;   // [QB][nword]
  int* pre;             // [QB][nword]
  unsigned int* uword;  // [nword]
  int* upre;            // [nword] exclusive prefix of the union popcounts (union step of each word)
  int* steps;           // [Sb / kTokSplit + 2] key blocks of this workgroup's union steps
  int* sinfo;           // [Sb / kTokSplit + 2] frame f and index u of each step's first key: (u << 8) | f
  int* s_w;             // [Nf] window w(t), clamped to N_t
  int* s_ret;           // [Nf] 1 iff t mod sf(t) = 0 (Eq. 6)
  int* prog;            // [kWaves] ring step each wave may still read (kDone: none)
  int* ready;           // [kRingMax] step held by each ring buffer (-1: none)
  unsigned char* rest;  // 16-byte aligned
  __host__ __device__ static size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }
  __device__ unsigned char* kbuf(int j) const { return ring + (j % nb) * G::KBUF; }
  __host__ __device__ static int max_steps(int Sb) { return Sb / kTokSplit + 2; }
  __device__ Lds(unsigned char* smem, int Sb, int Nf, int nb_) {
    nword = (Sb + 31) >> 5;
    nb = nb_;
    ring = smem;
    bits = reinterpret_cast<unsigned int*>(smem + (size_t)nb * G::KBUF);
    pre = reinterpret_cast<int*>(bits + G::QB * nword);
    uword = reinterpret_cast<unsigned int*>(pre + G::QB * nword);
    upre = reinterpret_cast<int*>(uword + nword);
    steps = upre + nword;
    sinfo = steps + max_steps(Sb);
    s_w = sinfo + max_steps(Sb);
    s_ret = s_w + Nf;
    prog = reinterpret_cast<int*>(smem + align16((size_t)(reinterpret_cast<unsigned char*>(s_ret + Nf) - smem)));
    ready = prog + kWaves;
    rest = reinterpret_cast<unsigned char*>(prog) + kCtlBytes;
  }
  __host__ __device__ static size_t bytes(int Sb, int Nf, int nb) {
    const size_t nw = (size_t)(Sb + 31) / 32;
    const size_t used = (size_t)nb * G::KBUF + (size_t)G::QB * nw * 8 + nw * 8 + (size_t)max_steps(Sb) * 8 +
                        (size_t)Nf * 8;
    return ((used + 15) & ~(size_t)15) + kCtlBytes;
  }
};

// Mark-kernel LDS beyond the shared layout: thresholds (score and logit
// units) per frame pair, the column counts and arrivals per ring buffer (B_s > 32), and
// the split's flags.
template <int D, int BS, int HF>
__host__ __device__ size_t mark_extra(int Sb, int Nf, int FR, int nb) {
  using G = Geo<D, BS, HF>;
  return (size_t)FR * Nf * 8 + (G::WPQ > 1 ? (size_t)G::QB * nb * (BS + 1) * 4 : 0) +
         (size_t)G::QB * Lds<D, BS, HF>::max_steps(Sb);
}

// First union step of key-range split `split` (kTokSplit workgroups share one
// query group's walk, each taking a contiguous run of its steps).
__device__ __forceinline__ int step_begin(int nsteps, int split) {
  return (int)(((long long)nsteps * split) / kTokSplit);
}

// The key-block ring without workgroup barriers. Loader wavefront l copies
// the steps l, l + kLoadWaves, ... of the split in order, one step in flight:
// before issuing a step it waits (s_waitcnt vmcnt) for its previous step's
// copies and publishes that step, then waits until the step's buffer is free
// (every compute wave past the step the buffer held, and that step
// published: a step no wave needs could otherwise still be landing). Compute
// waves walk only the steps their own query block needs: announce the step,
// wait until it is published, read. Waits are bounded.
template <int D, int BS, int HF>
__device__ __forceinline__ void ring_load(const TokParams& p, int b, const Lds<D, BS, HF>& L, int n, int l, int lane) {
  bool gave_up = false;
  int prev = -1;
  for (int j = l; j < n; j += kLoadWaves) {
    if (prev >= 0) {
      wait_vmcnt<0>();
      compiler_fence();
      st_relaxed(&L.ready[prev % L.nb], prev);
    }
    int spins = 0;
    while (true) {
      // explicit LDS loads (a generic load would also wait for copies in flight)
      const volatile DR_LDS intx4* pv = (const volatile DR_LDS intx4*)(L.prog);
      const intx4 a = pv[0];
      const intx4 c = pv[1];
      const int mn = uniform(min(min(min(a[0], a[1]), min(a[2], a[3])), min(min(c[0], c[1]), min(c[2], c[3]))));
      const bool free_buf =
          mn >= j - L.nb + 1 && (j < L.nb || uniform(ld_relaxed(&L.ready[j % L.nb])) == j - L.nb);
      if (free_buf) break;
      if (++spins > p.spin_limit) {
        gave_up = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    compiler_fence();
    __builtin_amdgcn_s_setprio(2);
    issue_block<D, BS, HF>(p, b, uniform(L.steps[j]), L.kbuf(j), lane);
    __builtin_amdgcn_s_setprio(0);
    prev = j;
  }
  if (prev >= 0) {
    wait_vmcnt<0>();
    compiler_fence();
    st_relaxed(&L.ready[prev % L.nb], prev);
  }
  if (gave_up && lane == 0) atomicOr(&g_tok_wait_flags, kWaitToken);
}

// Announce step j, then wait until its key block is in the ring.
template <int D, int BS, int HF>
__device__ __forceinline__ void ring_wait(const TokParams& p, const Lds<D, BS, HF>& L, int wave, int lane, int j,
                                          bool& gave_up) {
  compiler_fence();
  st_relaxed(&L.prog[wave], j);
  int spins = 0;
  while (ld_relaxed(&L.ready[j % L.nb]) != j) {
    if (++spins > p.spin_limit) {
      gave_up = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  compiler_fence();
}

// Leave the walk: no more reads.
template <int D, int BS, int HF>
__device__ __forceinline__ void ring_leave(const Lds<D, BS, HF>& L, int wave, int lane, bool gave_up) {
  compiler_fence();
  st_relaxed(&L.prog[wave], kDone);
  if (gave_up && lane == 0) atomicOr(&g_tok_wait_flags, kWaitToken);
}

// Visit the steps of this wave's query block (bitmap row `mine`) within the
// split's key range in ascending order: f(local step, key block).
template <int D, int BS, int HF, typename F>
__device__ __forceinline__ void walk_own(const Lds<D, BS, HF>& L, const unsigned int* mine, int n, int j0, F&& f) {
  if (n <= 0) return;
  const int kb_lo = L.steps[0], kb_hi = L.steps[n - 1];
  for (int wi = kb_lo >> 5; wi <= (kb_hi >> 5); ++wi) {
    unsigned int m = mine[wi];
    if (wi == (kb_lo >> 5)) m &= ~0u << (kb_lo & 31);
    if (wi == (kb_hi >> 5) && (kb_hi & 31) != 31) m &= (1u << ((kb_hi & 31) + 1)) - 1u;
    if (!m) continue;
    const unsigned int uw = L.uword[wi];
    const int up = L.upre[wi] - j0;
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      f(up + __popc(uw & ((1u << bit) - 1u)), wi * 32 + bit);
    }
  }
}

// Exclusive prefix sum over a wavefront (lane order); returns the total.
__device__ __forceinline__ int wave_scan(int c, int lane, int* excl) {
  int incl = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  *excl = incl - c;
  return __shfl(incl, 63);
}

// Setup shared by the stats and mark kernels: the per-distance table, the
// candidate bitmaps of the workgroup's query blocks with their CSR word
// prefixes, the union bitmap, and the key blocks of this split's union steps
// in ascending order. Returns their number.
template <int D, int BS, int HF>
__device__ __forceinline__ int setup(const TokParams& p, Lds<D, BS, HF>& L, int a0, int split, int* s_nsteps) {
  using G = Geo<D, BS, HF>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < kWaves) L.prog[tid] = 0;
  if (tid < kRingMax) L.ready[tid] = -1;
  for (int t = tid; t < p.Nf; t += kThreads) {
    int w, sf;
    table_entry(t, p.Nt, BS, p.L0, p.gamma, p.lambda, &w, &sf);
    L.s_w[t] = w < p.Nt ? w : p.Nt;
    L.s_ret[t] = t % sf == 0 ? 1 : 0;
  }
  for (int i = tid; i < G::QB * L.nword; i += kThreads) L.bits[i] = 0;
  __syncthreads();
  for (int qb = wave; qb < G::QB; qb += kWaves) {
    const int a = a0 + qb;
    if (a >= p.Sb) continue;
    const int e1 = p.row_ptr[a + 1];
    for (int e = p.row_ptr[a] + lane; e < e1; e += 64) {
      const int c = p.cols[e];
      atomicOr(&L.bits[qb * L.nword + (c >> 5)], 1u << (c & 31));
    }
  }
  __syncthreads();
  for (int wi = tid; wi < L.nword; wi += kThreads) {
    unsigned int u = 0;
    for (int s = 0; s < G::QB; ++s) u |= L.bits[s * L.nword + wi];
    L.uword[wi] = u;
  }
  // per query block: exclusive popcount prefix over its words (CSR positions)
  for (int qb = wave; qb < G::QB; qb += kWaves) {
    int run = 0;
    for (int w0 = 0; w0 < L.nword; w0 += 64) {
      const int wi = w0 + lane;
      int excl;
      const int tot = wave_scan(wi < L.nword ? __popc(L.bits[qb * L.nword + wi]) : 0, lane, &excl);
      if (wi < L.nword) L.pre[qb * L.nword + wi] = run + excl;
      run += tot;
    }
  }
  __syncthreads();
  if (wave == 0) {
    int run = 0;
    for (int w0 = 0; w0 < L.nword; w0 += 64) {
      const int wi = w0 + lane;
      int excl;
      const int tot = wave_scan(wi < L.nword ? __popc(L.uword[wi]) : 0, lane, &excl);
      if (wi < L.nword) L.upre[wi] = run + excl;
      run += tot;
    }
    if (lane == 0) *s_nsteps = run;
  }
  __syncthreads();
  const int nsteps = *s_nsteps;
  const int j0 = step_begin(nsteps, split), j1 = step_begin(nsteps, split + 1);
  for (int wi = tid; wi < L.nword; wi += kThreads) {
    unsigned int u = L.uword[wi];
    int j = L.upre[wi];
    if (j >= j1 || j + __popc(u) <= j0) continue;
    for (; u != 0u; u &= u - 1u, ++j)
      if (j >= j0 && j < j1) {
        const int kb = wi * 32 + __ffs(u) - 1;
        const int k0 = kb * BS, fk = k0 / p.Nt;
        L.steps[j - j0] = kb;
        L.sinfo[j - j0] = ((k0 - fk * p.Nt) << 8) | fk;
      }
  }
  __syncthreads();
  return j1 - j0;
}

// ---------------------------------------------------------------------------
// Pass 1: per-frame-pair statistics of the t > 1 candidate pairs.
// ---------------------------------------------------------------------------
template <int D, int BS, int HF>
__global__ __launch_bounds__(kThreads) void stats_kernel(TokParams p) {
  using G = Geo<D, BS, HF>;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_nsteps;
  Lds<D, BS, HF> L(smem, p.Sb, p.Nf, p.nb);
  Stat* acc_l = reinterpret_cast<Stat*>(L.rest);     // [kWaves][2][Nf]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int wg = blockIdx.x / kTokSplit, split = blockIdx.x - wg * kTokSplit, b = blockIdx.y;
  const int a0 = wg * G::QB;
  for (int i = tid; i < kWaves * 2 * p.Nf; i += kThreads) acc_l[i] = Stat{0.0, 0.0, 0.0, 0ull};
  const int n = setup<D, BS, HF>(p, L, a0, split, &s_nsteps);

  const int qb = wave / G::WPQ, sub = wave - qb * G::WPQ;
  const int a = a0 + qb;
  const int q0 = a * BS + 32 * sub;
  const bool active_wave = wave < kWaves && a < p.Sb && q0 < p.S;
  bf16x8 qf[HF][D / 16];
  if (active_wave) load_q<D, HF>(p, b, q0, lane, qf);
  wait_vmcnt<0>();
  const int f0w = q0 / p.Nt;
  const FrameAt qat{f0w, q0 - f0w * p.Nt};   // frame and index of the wave's first row
  Stat* mine = acc_l + wave * 2 * p.Nf;
  // B_s <= 64: candidate entry of the wave's current step. The walk visits the
  // wave's candidates in ascending key order, one entry after another, from
  // the first at or after the split's first step.
  int entry = 0;
  if (BS <= kDecideMaxBs && active_wave && n > 0) {
    const int kb = L.steps[0], wi = kb >> 5;
    entry = uniform(p.row_ptr[a] + L.pre[qb * L.nword + wi] +
                    __popc(L.bits[qb * L.nword + wi] & ((1u << (kb & 31)) - 1u)));
  }

  // Per-lane running statistics, 2 * NF sets: query frame f0w + fo (fo < NF;
  // NF = 2 only for a wave whose 32 rows cross a frame boundary, so that the
  // other waves keep half the state and stay within the register budget) x key
  // frame parity kp. Keys are walked in ascending order and the 32 keys of a
  // tile span at most two adjacent frames, so the set of parity kp holds one key
  // frame (tag0 / tag1) at a time; it is reduced over the wave and merged into
  // the wave's LDS statistics once the walk has passed that frame. Per tile, a
  // lane sums its (at most 16) logits and their squares in float32; the set adds
  // those tile sums, scaled, as float64 power sums. The highest score keeps its
  // position for safeguard (ii).
  const int j0 = step_begin(s_nsteps, split);
  bool gave_up = false;
  if (wave >= kWaves) ring_load<D, BS, HF>(p, b, L, n, wave - kWaves, lane);
  auto run = [&](auto nf_tag) {
    constexpr int NF = decltype(nf_tag)::value, NS = 2 * NF;
    double rs[NS], rq[NS];
    int rn[NS];
    float rm[NS];
    unsigned int rl[NS];
#pragma unroll
    for (int x = 0; x < NS; ++x) {
      rs[x] = rq[x] = 0.0;
      rn[x] = 0;
      rm[x] = -INFINITY;
      rl[x] = 0xffffffffu;
    }
    int tag0 = -1, tag1 = -1;   // key frame held by the parity-0 / parity-1 sets
    auto tag_of = [&](int kp) -> int { return kp ? tag1 : tag0; };
    auto set_tag = [&](int kp, int f) {
      if (kp) tag1 = f;
      else tag0 = f;
    };
    auto flush = [&](int kp) {
      if (tag_of(kp) < 0) return;
#pragma unroll
      for (int fo = 0; fo < NF; ++fo) {
        const int x = 2 * fo + kp;
        int cnt = rn[x];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
        if (cnt > 0) {
          const double sum = wave_sum(rs[x]), sq = wave_sum(rq[x]);
          const unsigned long long mx = wave_max(rl[x] == 0xffffffffu ? 0ull : pack_max(rm[x], rl[x]));
          const double nn = (double)cnt, mean = sum / nn;
          double m2 = sq - sum * mean;
          if (m2 < 0.0) m2 = 0.0;
          if (lane == 0) merge(mine[fo * p.Nf + tag_of(kp)], nn, mean, m2, mx);
        }
        rs[x] = rq[x] = 0.0;
        rn[x] = 0;
        rm[x] = -INFINITY;
        rl[x] = 0xffffffffu;
      }
      set_tag(kp, -1);
    };
    // add a lane's tile sums to set x (x may differ between lanes)
    auto add = [&](int x, double ts, double tq, int tn, float tm, unsigned int tl) {
#pragma unroll
      for (int y = 0; y < NS; ++y)
        if (y == x) {
          rs[y] += ts;
          rq[y] += tq;
          rn[y] += tn;
          if (tm > rm[y] || (tm == rm[y] && tl < rl[y])) {
            rm[y] = tm;
            rl[y] = tl;
          }
        }
    };

    // key blocks stream through the LDS ring; a compute wave visits only its own
    if (active_wave) {
      walk_own(L, L.bits + qb * L.nword, n, j0, [&](int j, int kb) __attribute__((always_inline)) {
        const int ent = entry++;
        ring_wait<D, BS, HF>(p, L, wave, lane, j, gave_up);
        const unsigned char* kbuf = L.kbuf(j);
        const int info = L.sinfo[j];
        const FrameAt kat0{info & 255, info >> 8};
  #pragma unroll 1
        for (int ksub = 0; ksub < BS / 32; ++ksub) {
          const int ktok0 = kb * BS + 32 * ksub;
          if (ktok0 >= p.S) break;
          const FrameAt kat = frame_after(kat0, 32 * ksub, p.Nt);
          const TileInfo ti = classify(p, q0, qat, ktok0, kat, L.s_w, L.s_ret);
          if (ti.cls == kNone || ti.cls == kAllNear) continue;      // no t > 1 pair of P
          // retire the sets whose key frame the walk has passed
          const int fk_first = kat.f;
  #pragma unroll
          for (int kp = 0; kp < 2; ++kp)
            if (tag_of(kp) >= 0 && tag_of(kp) < fk_first) flush(kp);
          const floatx16 acc = tile_scores<D, BS, HF>(qf, kbuf, ksub, lane);
          if (ti.cls == kAllScored) {
            // all 1024 pairs in P(fq, fk): one set, no masks. Sums of the lane's
            // 16 logits in float32, scaled into the float64 set; the scale is
            // positive, so the tile maximum scales to the maximum score.
            set_tag(ti.fk & 1, ti.fk);
            const int x = 2 * (ti.fq - f0w) + (ti.fk & 1);
            float ts = 0.f, tq = 0.f, m = -INFINITY;
  #pragma unroll
            for (int i = 0; i < 16; ++i) {
              ts += acc[i];
              tq = fmaf(acc[i], acc[i], tq);
              m = fmaxf(m, acc[i]);
            }
            // the tile's key-column sums for the decision pass (B_s <= 64): lanes
            // l and l ^ 32 hold the two 16-row halves of column l % 32
            const float cs = sum_halves(ts), cq = sum_halves(tq);
            const float ms = m * p.scale;
            float cur = rm[0];
#pragma unroll
            for (int y = 1; y < NS; ++y)
              if (x == y) cur = rm[y];
            unsigned int loc = 0xffffffffu;
            if (__ballot(ms >= cur) != 0ull) {
              // first of the lane's rows reaching m: rows ascend with i, and so
              // does the position u * N_t + v
              int first = 15;
  #pragma unroll
              for (int i = 15; i >= 0; --i)
                if (acc[i] == m) first = i;
              loc = (unsigned)((qat.u + row_of(first, half)) * p.Nt + (kat.u + (lane & 31)));
            }
            const double sc = (double)p.scale;
            add(x, (double)ts * sc, (double)tq * (sc * sc), 16, ms, loc);
            if constexpr (BS <= kDecideMaxBs) {
              // stored after the set update: spill reloads there would wait for
              // every memory operation in flight, this store included
              compiler_fence();
              if (lane < 32) colsum_of<BS>(p, b, ent, sub, ksub)[lane] = floatx2{cs, cq};
            }
            continue;
          }
          // general tile: pairs split by query frame f0 + fo and the lane's key frame
          const TileFrames f = tile_frames_at(p, qat, kat, ktok0, lane);
          set_tag(fk_first & 1, fk_first);
          if (kat.u + min(31, p.S - 1 - ktok0) >= p.Nt) set_tag((fk_first + 1) & 1, fk_first + 1);
          const int t0 = f.f0 > f.fk ? f.f0 - f.fk : f.fk - f.f0;
          const int t1 = f.f0 + 1 > f.fk ? f.f0 + 1 - f.fk : f.fk - f.f0 - 1;
          const bool ok0 = f.kvalid && t0 > 1 && t0 < p.Nf && L.s_ret[t0];
          const bool ok1 = f.kvalid && t1 > 1 && t1 < p.Nf && L.s_ret[t1];
          const int w0 = t0 < p.Nf ? L.s_w[t0] : 0, w1 = t1 < p.Nf ? L.s_w[t1] : 0;
          // per query frame f0 (suffix 0) and f0 + 1 (suffix 1); scalars, so that
          // a lane-dependent choice never indexes memory
          float ts0 = 0.f, tq0 = 0.f, ts1 = 0.f, tq1 = 0.f;
          int tn0 = 0, tn1 = 0;
          float tm0 = -INFINITY, tm1 = -INFINITY;
          unsigned int tl0 = 0xffffffffu, tl1 = 0xffffffffu;
  #pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = row_of(i, half);
            if (q0 + r >= p.S) continue;
            int u = f.u0 + r;
            const bool second = u >= p.Nt;
            if (second) u -= p.Nt;
            const int du = u > f.uk ? u - f.uk : f.uk - u;
            if (!(second ? (ok1 && du <= w1) : (ok0 && du <= w0))) continue;
            const float a = acc[i];
            const float v = a * p.scale;
            const unsigned int loc = (unsigned)(u * p.Nt + f.uk);
            // rows ascend with i: the first maximum has the lowest position
            if (second) {
              ts1 += a;
              tq1 = fmaf(a, a, tq1);
              ++tn1;
              if (v > tm1) {
                tm1 = v;
                tl1 = loc;
              }
            } else {
              ts0 += a;
              tq0 = fmaf(a, a, tq0);
              ++tn0;
              if (v > tm0) {
                tm0 = v;
                tl0 = loc;
              }
            }
          }
          const int kp = f.fk & 1;
          const double sc = (double)p.scale;
          if (tn0 > 0) add(kp, (double)ts0 * sc, (double)tq0 * (sc * sc), tn0, tm0, tl0);
          if constexpr (NF == 2) {
            if (tn1 > 0) add(2 + kp, (double)ts1 * sc, (double)tq1 * (sc * sc), tn1, tm1, tl1);
          }
          if constexpr (BS <= kDecideMaxBs) {
            if (ti.cls == kCutScored || key_straddle(p, q0, qat, ktok0, ti)) {
              // the rows lie in one query frame and each key column in one frame
              // pair (a tile cut by the window, or whose keys cross a frame
              // boundary): the columns' in-P sums for the decision pass (after
              // the set update, as above)
              const float cs = sum_halves(ts0), cq = sum_halves(tq0);
              compiler_fence();
              if (lane < 32) colsum_of<BS>(p, b, ent, sub, ksub)[lane] = floatx2{cs, cq};
            }
          }
        }
      });
    }
    if (wave < kWaves) ring_leave(L, wave, lane, gave_up);
    flush(0);
    flush(1);
  };
  if (active_wave && qat.u + 31 >= p.Nt) run(std::integral_constant<int, 2>{});
  else run(std::integral_constant<int, 1>{});
  __syncthreads();
  // merge the waves in order into the workgroup partial: [FR][Nf] per workgroup
  const int f_lo = (a0 * BS) / p.Nt;
  for (int i = tid; i < p.FR * p.Nf; i += kThreads) {
    const int fr = i / p.Nf, fk = i - fr * p.Nf;
    Stat t{0.0, 0.0, 0.0, 0ull};
    for (int w = 0; w < kWaves; ++w) {
      const int qbw = w / G::WPQ, subw = w - qbw * G::WPQ;
      const int q0w = (a0 + qbw) * BS + 32 * subw;
      if (a0 + qbw >= p.Sb || q0w >= p.S) continue;
      const int fo = f_lo + fr - q0w / p.Nt;
      if (fo < 0 || fo > 1) continue;
      const Stat& m = acc_l[(w * 2 + fo) * p.Nf + fk];
      merge(t, m.n, m.mean, m.m2, m.mx);
    }
    Stat* out = p.part + (((size_t)(b * p.n_wg + wg) * kTokSplit + split) * p.FR + fr) * p.Nf + fk;
    *out = t;
  }
}

// ---------------------------------------------------------------------------
// Pass 2: per frame pair, merge the workgroup partials (in order) and derive
// the threshold in score units.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void reduce_kernel(TokParams p) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  if (i >= p.Nf * p.Nf) return;
  const int fq = i / p.Nf, fk = i - fq * p.Nf;
  Stat t{0.0, 0.0, 0.0, 0ull};
  const int w_lo = (int)(((long long)fq * p.Nt) / kRows);
  const int w_hi = (int)(((long long)(fq + 1) * p.Nt - 1) / kRows);
  for (int w = w_lo; w <= w_hi && w < p.n_wg; ++w) {
    const int f_lo = (int)(((long long)w * kRows) / p.Nt);
    const int fr = fq - f_lo;
    if (fr < 0 || fr >= p.FR) continue;
    for (int sp = 0; sp < kTokSplit; ++sp) {
      const Stat& m = p.part[(((size_t)(b * p.n_wg + w) * kTokSplit + sp) * p.FR + fr) * p.Nf + fk];
      merge(t, m.n, m.mean, m.m2, m.mx);
    }
  }
  float thr = INFINITY;
  if (t.n > 0.0) {
#pragma clang fp contract(off)
    const int dt = fq > fk ? fq - fk : fk - fq;
    const int B = 32 - __builtin_clz((unsigned)dt);
    const double decay = (double)p.L0 / (double)(1LL << B) * p.gamma;   // Eq. 2
    const double tau = decay >= (double)p.Bs ? p.tau_near : p.tau_far;  // Eq. 11
    const double sigma = sqrt(t.m2 / t.n);
    const double bound = t.mean + tau * (sigma + p.eps);
    // smallest float >= bound (float32 s >= it  <=>  (double) s >= bound)
    float f = (float)bound;
    if ((double)f < bound) f = nextafterf(f, INFINITY);
    thr = f;
  }
  const size_t o = (size_t)b * p.Nf * p.Nf + i;
  p.thr[o] = thr;
  p.fmax[o] = t.mx;
  p.fn[o] = t.n;
  // served iff some pair of P(i, j) reaches the threshold, i.e. iff its
  // highest score does (the same float32 scores the mark pass compares; fkey
  // preserves order)
  p.served[o] = t.n > 0.0 && (unsigned int)(t.mx >> 32) >= fkey(thr) ? 1 : 0;
}

// The smallest float a with fl(a * scale) >= thr (scale > 0): rounding is
// monotone, so for every float x, x >= a exactly when fl(x * scale) >= thr.
// thr / scale lies within two ulps of it; +-inf map to themselves.
__device__ __forceinline__ float logit_threshold(float thr, float scale) {
  if (__builtin_isinf(thr)) return thr;
  float a = thr / scale;
  for (int it = 0; it < 4; ++it) {
    const float d = nextafterf(a, -INFINITY);
    if (d * scale >= thr) a = d;
    else break;
  }
  for (int it = 0; it < 4 && !(a * scale >= thr); ++it) a = nextafterf(a, INFINITY);
  return a;
}

// Decision of one block pair from per-key-token selected counts.
__device__ __forceinline__ bool block_kept(const TokParams& p, const int* cnt, int nq, int nk) {
  int act = 0;
  for (int c = 0; c < nk; ++c) act += ((double)cnt[c] / (double)nq) > p.theta_c ? 1 : 0;
  return ((double)act / (double)nk) > p.theta_m;
}

// ---------------------------------------------------------------------------
// Pass 3a (B_s <= 64): candidate entries whose flag follows without their
// logits. When a block's query rows lie in one frame (and it stays clear of
// the sequence end), each key column lies in one frame pair (also when the
// keys cross a frame boundary), and its selected count is known outright if
// that pair has t <= 1 (its in-window rows) or no pair in P (none). For t > 1,
// Cantelli's inequality bounds the count of the column's n in-window logits
// (over the block's 32-row tiles, whose column sums add)
// at or above the logit threshold T: at most n v / (v + d^2) of them lie d or
// more above their mean (v: population variance), and as many at most d or
// more below it. Mean and variance come from the statistics pass's float32
// column sums, widened by their rounding bounds (a float32 sum of n terms is
// within (n + 1) u sum |x| of the exact one, a fused sum of squares within
// (n + 1) u sum x^2; 20 u is taken), so a column fixed as active (count >=
// the theta_c count) or inactive is so for its logits, and the flag is fixed
// once enough columns are. Exact: a fixed flag is the flag the mark pass would
// compute. The other entries (und = 1: query rows crossing a frame boundary,
// the sequence end, columns the bound leaves open) go to mark_open_kernel.
// One workgroup per (b, query block), B_s lanes per entry (lane = key column).
// ---------------------------------------------------------------------------
template <int D, int BS, int HF>
__global__ __launch_bounds__(256) void decide_kernel(TokParams p) {
  static_assert(BS == 32 || BS == 64, "a block pair's key columns on one lane group");
  constexpr int QS = BS / 32;           // 32-row (and 32-key) sub-tiles per side
  constexpr int EPW = 64 / BS;          // entries per wavefront (lane group = BS lanes)
  constexpr int GROUPS = 256 / BS;      // lane groups per workgroup
  __shared__ int s_w[kMaxTokenFrames], s_ret[kMaxTokenFrames];
  __shared__ float s_thra[kMaxTokenFrames];   // logit threshold against key frame fk
  const int tid = threadIdx.x, lane = tid & 63, col = tid % BS, grp = tid / BS;
  const int a = blockIdx.x, b = blockIdx.y;
  const int q0 = a * BS;
  const FrameAt qat{q0 / p.Nt, q0 - (q0 / p.Nt) * p.Nt};
  for (int t = tid; t < p.Nf; t += 256) {
    int w, sf;
    table_entry(t, p.Nt, BS, p.L0, p.gamma, p.lambda, &w, &sf);
    s_w[t] = w < p.Nt ? w : p.Nt;
    s_ret[t] = t % sf == 0 ? 1 : 0;
    s_thra[t] = logit_threshold(p.thr[((size_t)b * p.Nf + qat.f) * p.Nf + t], p.scale);
  }
  __syncthreads();
  const int min_c = min_count(BS, p.theta_c), min_a = min_count(BS, p.theta_m);
  const int e0 = p.row_ptr[a], e1 = p.row_ptr[a + 1];
  const size_t eb = (size_t)b * p.nnz;
  const unsigned long long gmask = EPW == 1 ? ~0ull : ((lane >> 5) ? 0xffffffff00000000ull : 0xffffffffull);
  // every row of the block valid and in frame qat.f
  const bool rows_one_frame = q0 + BS - 1 < p.S && qat.u + BS - 1 < p.Nt;
  const int ksub = col >> 5, c32 = col & 31;   // this lane's key sub-block and column in it
  // kDecideUnroll entries per lane group in flight: their loads first
  for (int base = e0 + grp; base - grp < e1; base += GROUPS * kDecideUnroll) {
    int k0s[kDecideUnroll];
    floatx2 sums[kDecideUnroll][QS];
#pragma unroll
    for (int j = 0; j < kDecideUnroll; ++j) {
      const int e = base + GROUPS * j;
      k0s[j] = e < e1 ? p.cols[e] * BS : p.S;
      // read whether or not the entry needs them: unused values are discarded
#pragma unroll
      for (int sub = 0; sub < QS; ++sub)
        sums[j][sub] = e < e1 ? colsum_of<BS>(p, b, e, sub, ksub)[c32] : floatx2{0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < kDecideUnroll; ++j) {
      const int e = base + GROUPS * j;
      const bool valid = e < e1;
      const int k0 = k0s[j];
      // the block's query rows lie in frame qat.f; each key column of it in
      // one key frame fk (its keys may cross one frame boundary, N_t >= B_s)
      const bool open_tile = !(valid && rows_one_frame && k0 + BS - 1 < p.S);
      bool act = false, inact = false;
      if (!open_tile) {
        const int kt = k0 + col;
        const int fk = kt / p.Nt, v = kt - fk * p.Nt;
        // the column's pairs in P(qat.f, fk): its in-window rows, if retained,
        // per 32-row sub-tile
        const int t = qat.f > fk ? qat.f - fk : fk - qat.f;
        const int w = s_w[t];
        int nin = 0, nsub[QS];
#pragma unroll
        for (int sub = 0; sub < QS; ++sub) {
          const int u0 = qat.u + 32 * sub;
          nsub[sub] = s_ret[t] ? max(0, min(u0 + 31, v + w) - max(u0, v - w) + 1) : 0;
          nin += nsub[sub];
        }
        if (t <= 1 || nin == 0) {
          // all of them selected (t <= 1), or none exist
          act = (t <= 1 ? nin : 0) >= min_c;
          inact = !act;
        } else {
          // with n values, mean m, population variance var and the threshold T:
          // M = n Qhi - sa^2 >= n^2 var, dn = n (T - m) or n (m - T) less e1s;
          // the Cantelli tests n var / (var + d^2) < min_c and
          // n d^2 / (var + d^2) > min_c - 1 multiplied through by n^2 (var + d^2).
          // A sub-tile's sums exist wherever it has in-window rows (the
          // statistics pass stores them for every such tile).
          const double n = (double)nin, u = 0x1p-24;
          double S1 = 0.0, Q = 0.0;
#pragma unroll
          for (int sub = 0; sub < QS; ++sub)
            if (nsub[sub] > 0) {
              S1 += (double)sums[j][sub][0];
              Q += (double)sums[j][sub][1];
            }
          const double T = s_thra[fk];
          const double Qhi = Q * (1.0 + 20.0 * u);                               // >= the exact sum of squares
          const double e1s = 20.0 * u * (double)sqrtf((float)(n * Qhi)) * (1.0 + 1e-6);  // >= |S1 - the exact sum|
          const double sa = fmax(0.0, fabs(S1) - e1s);
          const double M = fmax(0.0, n * Qhi - sa * sa);
          const double A = n * T - S1;                                             // n (T - m), within e1s
          if (__builtin_isfinite(T) && A - e1s > 0.0) {
            const double dn = A - e1s;
            inact = n * M * (1.0 + 1e-12) < (double)min_c * (M + dn * dn);
          } else if (__builtin_isfinite(T) && -A - e1s > 0.0) {
            const double dn = -A - e1s;
            act = n * dn * dn * (1.0 - 1e-12) > (double)(min_c - 1) * (M + dn * dn);
          }
        }
      }
      const int n_act = __popcll(__ballot(act) & gmask), n_in = __popcll(__ballot(inact) & gmask);
      const bool decided = !open_tile && (n_act >= min_a || BS - n_in < min_a);
      if (valid && col == 0) {
        if (decided) p.flags[eb + e] = n_act >= min_a ? 1 : 0;
        p.und[eb + e] = decided ? 0 : 1;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Pass 3b (B_s <= 64): the entries the decision pass left open, decided as the
// mark pass below decides them. Few stay open (1.4% at wan14b_720p + "mid",
// 2.5% at hunyuan_720p: every entry of a query block that straddles two
// frames, the sequence end, columns the bound leaves open), so there is no
// staging ring: one wavefront per
// kOpenChunk consecutive candidate entries (rows with many open entries are
// spread over many wavefronts) loads its query block's fragments and reads
// each open entry's key fragments straight from memory. Served frame pairs
// are already final (reduce kernel).
// ---------------------------------------------------------------------------
template <int D, int BS, int HF>
__global__ __launch_bounds__(256) void mark_open_kernel(TokParams p) {
  constexpr int QS = BS / 32;           // 32-row (and 32-key) sub-tiles per side
  __shared__ int s_w[kMaxTokenFrames], s_ret[kMaxTokenFrames];
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, wave = tid >> 6;
  const int b = blockIdx.y;
  for (int t = tid; t < p.Nf; t += 256) {
    int w, sf;
    table_entry(t, p.Nt, BS, p.L0, p.gamma, p.lambda, &w, &sf);
    s_w[t] = w < p.Nt ? w : p.Nt;
    s_ret[t] = t % sf == 0 ? 1 : 0;
  }
  __syncthreads();
  // this wave's kOpenChunk consecutive candidate entries
  const long long c0 = ((long long)blockIdx.x * 4 + wave) * kOpenChunk;
  if (c0 >= p.nnz) return;
  const size_t eb = (size_t)b * p.nnz;
  unsigned long long open = __ballot(lane < kOpenChunk && c0 + lane < p.nnz && p.und[eb + c0 + lane] != 0);
  if (!open) return;
  // query block holding entry c0: the last a with row_ptr[a] <= c0
  int lo = 0, hi = p.Sb - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (uniform(p.row_ptr[mid]) <= c0) lo = mid;
    else hi = mid - 1;
  }
  int a = lo, a_end = uniform(p.row_ptr[a + 1]);
  const float* thr = p.thr + (size_t)b * p.Nf * p.Nf;
  bf16x8 qf[HF][D / 16];
  int q_loaded = -1;   // first row of the query fragments in registers
  while (open) {
    const long long e = c0 + __ffsll(open) - 1;
    open &= open - 1;
    while (e >= a_end) {
      ++a;
      a_end = uniform(p.row_ptr[a + 1]);
    }
    const int kb0 = uniform(p.cols[e]) * BS;
    const int nq = min(BS, p.S - a * BS), nk = min(BS, p.S - kb0);
    // selected count of key column 32 * ksub + lane % 32, summed over the
    // block's 32-row sub-tiles (both half-waves hold it)
    int cnt[QS];
#pragma unroll
    for (int ks = 0; ks < QS; ++ks) cnt[ks] = 0;
#pragma unroll 1
    for (int sub = 0; sub < QS; ++sub) {
      const int q0 = a * BS + 32 * sub;
      if (q0 >= p.S) break;
      if (q0 != q_loaded) {
        load_q<D, HF>(p, b, q0, lane, qf);
        q_loaded = q0;
      }
      const FrameAt qat{q0 / p.Nt, q0 - (q0 / p.Nt) * p.Nt};
#pragma unroll
      for (int ks = 0; ks < QS; ++ks) {
        const int k0 = kb0 + 32 * ks;
        if (k0 >= p.S) break;
        const FrameAt kat{k0 / p.Nt, k0 - (k0 / p.Nt) * p.Nt};
        const TileInfo ti = classify(p, q0, qat, k0, kat, s_w, s_ret);
        int c = ti.cls == kAllNear ? 32 : 0;
        if (ti.cls != kNone && ti.cls != kAllNear) {
          // key fragments of every fused head (rows past S read the last token;
          // those columns are outside P)
          const int key = min(k0 + (lane & 31), p.S - 1);
          floatx16 acc = {};
#pragma unroll
          for (int h = 0; h < HF; ++h) {
            const uint16_t* row = p.k + ((size_t)(b * p.H + h) * p.S + key) * D;
            bf16x8 kf[D / 16];
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
              kf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + (2 * kk + half) * 8));
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
              acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[h][kk], kf[kk], acc, 0, 0, 0);
          }
          if (ti.cls == kAllScored) {
            const float ta = logit_threshold(thr[ti.fq * p.Nf + ti.fk], p.scale);
            int below = 0;
#pragma unroll
            for (int i = 0; i < 16; ++i) below += (int)(__float_as_uint(acc[i] - ta) >> 31);
            c = 16 - below;
          } else {
            const TileFrames f = tile_frames_at(p, qat, kat, k0, lane);
            const float thr0 = f.kvalid ? thr[f.f0 * p.Nf + f.fk] : INFINITY;
            const float thr1 = (f.kvalid && f.f0 + 1 < p.Nf) ? thr[(f.f0 + 1) * p.Nf + f.fk] : INFINITY;
            unsigned sel, inP2;
            select_bits(p, acc, f, q0, half, s_w, s_ret, thr0, thr1, sel, inP2);
            c = __popc(sel);
          }
          c += __shfl_xor(c, 32);
        }
        cnt[ks] += c;
      }
    }
    // lane l decides key column l of the block (B_s = 64) or l % 32 (B_s = 32)
    const int c = QS == 1 ? cnt[0] : cnt[(lane >> 5) % QS];
    const int n_act = __popcll(__ballot(lane < nk && c >= min_count(nq, p.theta_c)));
    if (lane == 0) p.flags[eb + e] = n_act >= min_count(nk, p.theta_m) ? 1 : 0;
  }
}

// ---------------------------------------------------------------------------
// Pass 3: selection, aggregation to block pairs, one flag per candidate entry.
// ---------------------------------------------------------------------------
template <int D, int BS, int HF>
__global__ __launch_bounds__(kThreads) void mark_kernel(TokParams p) {
  using G = Geo<D, BS, HF>;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_nsteps;
  __shared__ int min_c[BS + 1], min_a[BS + 1], pos_lo[G::QB];
  Lds<D, BS, HF> L(smem, p.Sb, p.Nf, p.nb);
  const int MS = Lds<D, BS, HF>::max_steps(p.Sb);
  float* thr_l = reinterpret_cast<float*>(L.rest);                      // [FR][Nf]
  float* thra_l = thr_l + p.FR * p.Nf;                                  // [FR][Nf] in logit units
  int* colcnt = reinterpret_cast<int*>(thra_l + p.FR * p.Nf);           // [QB][nb][BS] when BS > 32
  int* arrive = colcnt + (G::WPQ > 1 ? G::QB * L.nb * BS : 0);           // [QB][nb] when BS > 32
  unsigned char* flags_l = reinterpret_cast<unsigned char*>(arrive + (G::WPQ > 1 ? G::QB * L.nb : 0));  // [QB][MS]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int wg = blockIdx.x / kTokSplit, split = blockIdx.x - wg * kTokSplit, b = blockIdx.y;
  const int a0 = wg * G::QB;
  const int f_lo = (a0 * BS) / p.Nt;
  if (G::WPQ > 1)
    for (int i = tid; i < G::QB * L.nb * (BS + 1); i += kThreads) colcnt[i] = 0;   // counts and arrivals
  for (int i = tid; i < p.FR * p.Nf; i += kThreads) {
    const int fr = i / p.Nf, fk = i - fr * p.Nf;
    const int fq = f_lo + fr;
    const float thr = fq < p.Nf ? p.thr[(size_t)b * p.Nf * p.Nf + (size_t)fq * p.Nf + fk] : INFINITY;
    thr_l[i] = thr;
    thra_l[i] = logit_threshold(thr, p.scale);
  }
  for (int n = 1 + tid; n <= BS; n += kThreads) {
    min_c[n] = min_count(n, p.theta_c);
    min_a[n] = min_count(n, p.theta_m);
  }
  const int n = setup<D, BS, HF>(p, L, a0, split, &s_nsteps);

  // position of key block kb in the candidate row of query block qb2
  auto pos_of = [&](int qb2, int kb) -> int {
    const int wi = kb >> 5;
    return L.pre[qb2 * L.nword + wi] + __popc(L.bits[qb2 * L.nword + wi] & ((1u << (kb & 31)) - 1u));
  };
  // this split's flags of row qb2 are kept in LDS from its first step on
  if (tid < G::QB && n > 0) pos_lo[tid] = pos_of(tid, L.steps[0]);

  const int qb = wave / G::WPQ, sub = wave - qb * G::WPQ;
  const int a = a0 + qb;
  const int q0 = a * BS + 32 * sub;
  const bool active_wave = wave < kWaves && a < p.Sb && q0 < p.S;
  const int nq = a < p.Sb ? min(BS, p.S - a * BS) : 0;
  const int n_sub = (nq + 31) / 32;   // waves of this query block holding rows
  const FrameAt qat{q0 / p.Nt, q0 - (q0 / p.Nt) * p.Nt};   // frame and index of the wave's first row
  bf16x8 qf[HF][D / 16];
  if (active_wave) load_q<D, HF>(p, b, q0, lane, qf);
  wait_vmcnt<0>();

  // selected count of key column lane % 32 of the tile (q0, ktok0) over the
  // wave's 32 query rows (the same value in both half-waves)
  auto tile_count = [&](const unsigned char* kbuf, int ksub, int ktok0, FrameAt kat) -> int {
    const TileInfo ti = classify(p, q0, qat, ktok0, kat, L.s_w, L.s_ret);
    if (ti.cls == kNone) return 0;
    if (ti.cls == kAllNear) return 32;
    const floatx16 acc = tile_scores<D, BS, HF>(qf, kbuf, ksub, lane);
    unsigned sel = 0;
    if (ti.cls == kAllScored) {
      // selected iff logit >= the frame pair's logit threshold: the sign bit
      // of their difference counts the rest (x - y is +0 when x = y)
      const float ta = thra_l[(ti.fq - f_lo) * p.Nf + ti.fk];
      int below = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) below += (int)(__float_as_uint(acc[i] - ta) >> 31);
      const int c = 16 - below;
      return c + __shfl_xor(c, 32);
    } else {
      const TileFrames f = tile_frames_at(p, qat, kat, ktok0, lane);
      const float thr0 = f.kvalid ? thr_l[(f.f0 - f_lo) * p.Nf + f.fk] : INFINITY;
      const float thr1 = (f.kvalid && f.f0 + 1 - f_lo < p.FR) ? thr_l[(f.f0 + 1 - f_lo) * p.Nf + f.fk] : INFINITY;
      unsigned inP2;
      select_bits(p, acc, f, q0, half, L.s_w, L.s_ret, thr0, thr1, sel, inP2);
    }
    const int c = __popc(sel);
    return c + __shfl_xor(c, 32);
  };

  // key blocks stream through the LDS ring; this wave visits only its own.
  // B_s > 32: the waves of a query block add their column counts in LDS (one
  // count row per ring buffer) and the last one to arrive decides.
  const int j0 = step_begin(s_nsteps, split);
  bool gave_up = false;
  if (wave >= kWaves) ring_load<D, BS, HF>(p, b, L, n, wave - kWaves, lane);
  if (active_wave) {
    walk_own(L, L.bits + qb * L.nword, n, j0, [&](int j, int kb) __attribute__((always_inline)) {
      ring_wait<D, BS, HF>(p, L, wave, lane, j, gave_up);
      const unsigned char* kbuf = L.kbuf(j);
      const int nk = min(BS, p.S - kb * BS);
      const int info = L.sinfo[j];
      const FrameAt kat0{info & 255, info >> 8};
      if (G::WPQ == 1) {
        // one wave holds the whole block pair: decide in registers
        const int c = tile_count(kbuf, 0, kb * BS, kat0);
        const int n_act = __popcll(__ballot(lane < nk && c >= min_c[nq]));
        if (lane == 0) flags_l[qb * MS + pos_of(qb, kb) - pos_lo[qb]] = n_act >= min_a[nk] ? 1 : 0;
      } else {
        int* cnt = colcnt + (qb * L.nb + j % L.nb) * BS;
#pragma unroll 1
        for (int ksub = 0; ksub < BS / 32; ++ksub) {
          const int ktok0 = kb * BS + 32 * ksub;
          if (ktok0 >= p.S) break;
          const int c = tile_count(kbuf, ksub, ktok0, frame_after(kat0, 32 * ksub, p.Nt));
          if (half == 0) atomicAdd(&cnt[32 * ksub + lane], c);
        }
        // LDS operations of a wave complete in order: its counts are in
        // before its arrival is counted
        int arrived = 0;
        if (lane == 0) arrived = atomicAdd(&arrive[qb * L.nb + j % L.nb], 1) + 1;
        if (uniform(arrived) == n_sub) {
          compiler_fence();
          int n_act = 0;
#pragma unroll
          for (int c0 = 0; c0 < BS; c0 += 64) {   // 64 key columns per pass
            const int col = c0 + lane;
            const int v = col < BS ? ld_relaxed(&cnt[col]) : 0;
            n_act += __popcll(__ballot(col < nk && v >= min_c[nq]));
            if (col < BS) cnt[col] = 0;
          }
          if (lane == 0) {
            flags_l[qb * MS + pos_of(qb, kb) - pos_lo[qb]] = n_act >= min_a[nk] ? 1 : 0;
            arrive[qb * L.nb + j % L.nb] = 0;
          }
        }
      }
    });
  }
  if (wave < kWaves) ring_leave(L, wave, lane, gave_up);
  __syncthreads();
  // write out this split's flags (a contiguous run of each candidate row)
  if (n > 0 && wave < G::QB && a0 + wave < p.Sb) {
    const int last = L.steps[n - 1];
    const int lo = pos_lo[wave];
    const int hi = pos_of(wave, last) + (int)((L.bits[wave * L.nword + (last >> 5)] >> (last & 31)) & 1u);
    unsigned char* out = p.flags + (long long)b * p.nnz + p.row_ptr[a0 + wave] + lo;
    for (int i = lane; i < hi - lo; i += 64) out[i] = flags_l[wave * MS + i];
  }
}

// ---------------------------------------------------------------------------
// Pass 4: safeguard (ii). One wavefront per frame pair (i, j) of batch b.
// ---------------------------------------------------------------------------
template <int D, int BS, int HF>
__global__ __launch_bounds__(64) void fallback_kernel(TokParams p) {
  using G32 = Geo<D, 32, HF>;   // one 32-key sub-block of all fused heads at a time
  __shared__ __align__(16) unsigned char kbuf[G32::KBUF];
  __shared__ int s_w[kMaxTokenFrames], s_ret[kMaxTokenFrames];
  __shared__ int cnt[BS];
  const int lane = threadIdx.x, half = lane >> 5;
  const int fp = blockIdx.x, b = blockIdx.y;
  const int fq = fp / p.Nf, fk = fp - fq * p.Nf;
  const size_t base = (size_t)b * p.Nf * p.Nf;
  auto unserved = [&](int i, int j) -> bool {
    if (i < 0 || j < 0 || i >= p.Nf || j >= p.Nf) return false;
    const size_t o = base + (size_t)i * p.Nf + j;
    return p.fn[o] > 0.0 && p.served[o] == 0;
  };
  if (!unserved(fq, fk)) return;
  // the highest-scoring pair of P(fq, fk)
  auto pair_of = [&](int i, int j, int* qt, int* kt) {
    const unsigned int loc = 0xffffffffu - (unsigned int)(p.fmax[base + (size_t)i * p.Nf + j] & 0xffffffffull);
    *qt = i * p.Nt + (int)(loc / (unsigned)p.Nt);
    *kt = j * p.Nt + (int)(loc % (unsigned)p.Nt);
  };
  int qt, kt;
  pair_of(fq, fk, &qt, &kt);
  const int a = qt / BS, kbk = kt / BS;
  // every unserved frame pair whose fallback pair lies in block pair (a, kbk);
  // the lowest-numbered one decides for all of them
  const int fa0 = (a * BS) / p.Nt, fa1 = (min(p.S, (a + 1) * BS) - 1) / p.Nt;
  const int fb0 = (kbk * BS) / p.Nt, fb1 = (min(p.S, (kbk + 1) * BS) - 1) / p.Nt;
  constexpr int kFramesPerBlock = BS / 32 + 1;   // frames a block can span (N_t >= 32)
  int extra_q[kFramesPerBlock * kFramesPerBlock], extra_k[kFramesPerBlock * kFramesPerBlock], n_extra = 0;
  for (int i = fa0; i <= fa1; ++i)
    for (int j = fb0; j <= fb1; ++j) {
      if (!unserved(i, j)) continue;
      int q2, k2;
      pair_of(i, j, &q2, &k2);
      if (q2 / BS != a || k2 / BS != kbk) continue;
      if (i * p.Nf + j < fp) return;   // a lower-numbered frame pair decides this block pair
      extra_q[n_extra] = q2;
      extra_k[n_extra] = k2;
      ++n_extra;
    }
  // the candidate entry of (a, kbk), if any (the aggregate of the selection
  // never exceeds that of P, so a non-candidate block pair stays dropped)
  int lo = p.row_ptr[a], hi = p.row_ptr[a + 1];
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (p.cols[mid] < kbk) lo = mid + 1; else hi = mid;
  }
  if (lo >= p.row_ptr[a + 1] || p.cols[lo] != kbk) return;
  for (int t = lane; t < p.Nf; t += 64) {
    int w, sf;
    table_entry(t, p.Nt, BS, p.L0, p.gamma, p.lambda, &w, &sf);
    s_w[t] = w < p.Nt ? w : p.Nt;
    s_ret[t] = t % sf == 0 ? 1 : 0;
  }
  for (int c = lane; c < BS; c += 64) cnt[c] = 0;
  for (int ksub = 0; ksub < BS / 32; ++ksub) {
    const int ktok0 = kbk * BS + 32 * ksub;
    if (ktok0 >= p.S) break;
    __syncthreads();   // the previous sub-block's reads are done
    for (int c = lane; c < HF * 32 * (D / 8); c += 64) {
      const int h = c / (32 * (D / 8));
      const int rem = c - h * (32 * (D / 8));
      const int key = rem / (D / 8), ch = rem - key * (D / 8);
      const int tok = ktok0 + key;
      u32x4 v = {0, 0, 0, 0};
      if (tok < p.S) v = *reinterpret_cast<const u32x4*>(p.k + ((size_t)(b * p.H + h) * p.S + tok) * D + ch * 8);
      *reinterpret_cast<u32x4*>(kbuf + (h * 32 + key) * G32::RB + ((ch ^ swz<D>(key)) << 4)) = v;
    }
    __syncthreads();
    for (int sub = 0; sub < BS / 32; ++sub) {
      const int q0 = a * BS + 32 * sub;
      if (q0 >= p.S) break;
      bf16x8 qf[HF][D / 16];
      load_q<D, HF>(p, b, q0, lane, qf);
      const floatx16 acc = tile_scores<D, 32, HF>(qf, kbuf, 0, lane);
      const TileFrames f = tile_frames(p, q0, ktok0 + (lane & 31));
      const float thr0 = f.kvalid ? p.thr[base + (size_t)f.f0 * p.Nf + f.fk] : INFINITY;
      const float thr1 = (f.kvalid && f.f0 + 1 < p.Nf) ? p.thr[base + (size_t)(f.f0 + 1) * p.Nf + f.fk] : INFINITY;
      unsigned sel, inP2;
      select_bits(p, acc, f, q0, half, s_w, s_ret, thr0, thr1, sel, inP2);
      const int ktok = ktok0 + (lane & 31);
      for (int e = 0; e < n_extra; ++e)
        if (extra_k[e] == ktok)
          for (int i = 0; i < 16; ++i)
            if (q0 + row_of(i, half) == extra_q[e]) sel |= 1u << i;
      int c = __popc(sel);
      c += __shfl_xor(c, 32);
      if (half == 0) cnt[32 * ksub + lane] += c;
    }
  }
  __syncthreads();
  if (lane == 0) {
    const int nq = min(BS, p.S - a * BS), nk = min(BS, p.S - kbk * BS);
    p.flags[(long long)b * p.nnz + lo] = block_kept(p, cnt, nq, nk) ? 1 : 0;
  }
}

// Pass 5 (ordered compaction of the flags into kept lists of every head) is
// flag_compact_kernel below.
// LDS of the stats and mark kernels with a ring of nb buffers, static arrays
// included; the larger of the two.
template <int D, int BS, int HF>
size_t lds_need(int Sb, int Nf, int FR, int nb) {
  using G = Geo<D, BS, HF>;
  const size_t base = Lds<D, BS, HF>::bytes(Sb, Nf, nb);
  const size_t stats = base + (size_t)kWaves * 2 * Nf * sizeof(Stat) + 16;
  const size_t mark = base + mark_extra<D, BS, HF>(Sb, Nf, FR, nb) + (size_t)(2 * (BS + 1) + G::QB) * 4 + 16;
  return stats > mark ? stats : mark;
}

// The deepest ring (at most kRingMax buffers) whose kernels fit in LDS; 0 if
// not even two buffers fit.
template <int D, int BS, int HF>
int ring_depth(int Sb, int Nf, int FR) {
  for (int nb = kRingMax; nb >= 2; --nb)
    if (lds_need<D, BS, HF>(Sb, Nf, FR, nb) <= (size_t)kTokLdsBytes) return nb;
  return 0;
}

// Whether the environment asks for the ring mark pass at every block size.
inline bool ring_mark_requested() {
  const char* v = std::getenv("DR_TOKEN_RING_MARK");
  return v && std::strcmp(v, "0") != 0 && v[0] != '\0';
}

// Pass 5 (ordered compaction of the flags into kept lists of every head) is
// flag_compact_kernel below.
template <int D, int BS, int HF>
hipError_t launch_all(TokParams p, int B, hipStream_t stream) {
  p.nb = ring_depth<D, BS, HF>(p.Sb, p.Nf, p.FR);
  if (p.nb < 2) return hipErrorInvalidValue;
  const size_t base = Lds<D, BS, HF>::bytes(p.Sb, p.Nf, p.nb);
  const size_t lds_stats = base + (size_t)kWaves * 2 * p.Nf * sizeof(Stat);
  const size_t lds_mark = base + mark_extra<D, BS, HF>(p.Sb, p.Nf, p.FR, p.nb);
  const dim3 grid((unsigned)(p.n_wg * kTokSplit), (unsigned)B);
  hipLaunchKernelGGL((stats_kernel<D, BS, HF>), grid, dim3(kThreads), lds_stats, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((p.Nf * p.Nf + 255) / 256), (unsigned)B), dim3(256), 0, stream,
                     p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // DR_TOKEN_RING_MARK=1 (a reference path for tests) runs the ring mark pass
  // at B_s <= 64 too: the decision and open-entry passes must give its flags
  bool ring = true;
  if constexpr (BS <= kDecideMaxBs) {
    if (!ring_mark_requested()) {
      ring = false;
      if (!p.colsum || !p.und) return hipErrorInvalidValue;
      hipLaunchKernelGGL((decide_kernel<D, BS, HF>), dim3((unsigned)p.Sb, (unsigned)B), dim3(256), 0, stream, p);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      const long long chunks = (p.nnz + kOpenChunk - 1) / kOpenChunk;
      hipLaunchKernelGGL((mark_open_kernel<D, BS, HF>), dim3((unsigned)((chunks + 3) / 4), (unsigned)B), dim3(256),
                         0, stream, p);
    }
  }
  if (ring) hipLaunchKernelGGL((mark_kernel<D, BS, HF>), grid, dim3(kThreads), lds_mark, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((fallback_kernel<D, BS, HF>), dim3((unsigned)(p.Nf * p.Nf), (unsigned)B), dim3(64), 0, stream,
                     p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const FlagCompact fc{p.row_ptr, p.cols, p.flags, p.nnz, p.nnz, p.Sb, p.H, p.kept_col, p.kept_cnt};
  return launch_flag_compact(fc, B, stream);
}

}  // namespace

// LDS the token selector needs at its shallowest ring (two buffers).
size_t token_lds_bytes(int D, int Bs, int Hf, int Sb, int Nf, int FR) {
  if (D == 128 && Bs == 128) return Hf == 1 ? lds_need<128, 128, 1>(Sb, Nf, FR, 2) : lds_need<128, 128, 2>(Sb, Nf, FR, 2);
  if (D == 64 && Bs == 128) return Hf == 1 ? lds_need<64, 128, 1>(Sb, Nf, FR, 2) : lds_need<64, 128, 2>(Sb, Nf, FR, 2);
  if (D == 128 && Bs == 32) return Hf == 1 ? lds_need<128, 32, 1>(Sb, Nf, FR, 2) : lds_need<128, 32, 2>(Sb, Nf, FR, 2);
  if (D == 128 && Bs == 64) return Hf == 1 ? lds_need<128, 64, 1>(Sb, Nf, FR, 2) : lds_need<128, 64, 2>(Sb, Nf, FR, 2);
  if (D == 64 && Bs == 32) return Hf == 1 ? lds_need<64, 32, 1>(Sb, Nf, FR, 2) : lds_need<64, 32, 2>(Sb, Nf, FR, 2);
  return Hf == 1 ? lds_need<64, 64, 1>(Sb, Nf, FR, 2) : lds_need<64, 64, 2>(Sb, Nf, FR, 2);
}

// One wavefront per (b, query block): flags -> ascending kept list, by ballots.
__global__ __launch_bounds__(256) void flag_compact_kernel(FlagCompact p) {
  const int lane = threadIdx.x & 63;
  const int a = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (a >= p.Sb) return;
  const int r0 = p.row_ptr[a], n = p.row_ptr[a + 1] - r0;
  const unsigned char* fl = p.flags + (long long)b * p.flag_stride + r0;
  int kept = 0;
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int i = i0 + lane;
    const bool keep = i < n && fl[i] != 0;
    const unsigned long long m = __ballot(keep);
    const int before = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0));
    if (keep) {
      const int col = p.cols[r0 + i];
      for (int h = 0; h < p.H; ++h) p.kept_col[(long long)(b * p.H + h) * p.nnz + r0 + kept + before] = col;
    }
    kept += __popcll(m);
  }
  if (lane == 0)
    for (int h = 0; h < p.H; ++h) p.kept_cnt[(long long)(b * p.H + h) * p.Sb + a] = kept;
}

hipError_t launch_flag_compact(const FlagCompact& c, int B, hipStream_t stream) {
  hipLaunchKernelGGL(flag_compact_kernel, dim3((unsigned)((c.Sb + 3) / 4), (unsigned)B), dim3(256), 0, stream, c);
  return hipGetLastError();
}

hipError_t take_wait_flags_token(unsigned* flags, hipStream_t stream) {
  unsigned v = 0;
  hipError_t e = hipMemcpyFromSymbolAsync(&v, HIP_SYMBOL(g_tok_wait_flags), sizeof v, 0, hipMemcpyDeviceToHost,
                                          stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e == hipSuccess && v != 0) {
    static const unsigned zero = 0;
    e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_tok_wait_flags), &zero, sizeof zero, 0, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
  }
  *flags = v;
  return e;
}

hipError_t launch_token_select(const TokParams& p, int B, int D, int Bs, int Hf, hipStream_t stream) {
  if (D == 128 && Bs == 32 && Hf == 1) return launch_all<128, 32, 1>(p, B, stream);
  if (D == 128 && Bs == 32 && Hf == 2) return launch_all<128, 32, 2>(p, B, stream);
  if (D == 128 && Bs == 64 && Hf == 1) return launch_all<128, 64, 1>(p, B, stream);
  if (D == 128 && Bs == 64 && Hf == 2) return launch_all<128, 64, 2>(p, B, stream);
  if (D == 64 && Bs == 32 && Hf == 1) return launch_all<64, 32, 1>(p, B, stream);
  if (D == 64 && Bs == 32 && Hf == 2) return launch_all<64, 32, 2>(p, B, stream);
  if (D == 64 && Bs == 64 && Hf == 1) return launch_all<64, 64, 1>(p, B, stream);
  if (D == 64 && Bs == 64 && Hf == 2) return launch_all<64, 64, 2>(p, B, stream);
  if (D == 128 && Bs == 128 && Hf == 1) return launch_all<128, 128, 1>(p, B, stream);
  if (D == 128 && Bs == 128 && Hf == 2) return launch_all<128, 128, 2>(p, B, stream);
  if (D == 64 && Bs == 128 && Hf == 1) return launch_all<64, 128, 1>(p, B, stream);
  if (D == 64 && Bs == 128 && Hf == 2) return launch_all<64, 128, 2>(p, B, stream);
  return hipErrorInvalidValue;
}

}  // namespace dr
