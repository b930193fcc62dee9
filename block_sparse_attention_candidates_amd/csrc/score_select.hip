// Block scoring and dual-mode selection on gfx950 ([DR] §3.2, block form;
// [DR] = "DynamicRad: Content-Adaptive Sparse Attention for Long Video
// Diffusion", arXiv 2604.20470).
//
//   pool:   one wavefront per (tensor, b, h, block): coalesced 16-byte bf16 loads
//           of the block's valid rows, float32 sums, cross-lane reduction, mean.
//           HBM-bound (reads Q and K once).
//   tiles:  one workgroup per group of 32 query blocks (head-independent): LDS
//           bitmaps of the 32 rows' candidates give every candidate's CSR
//           position; the active 32x32 tiles and their bitmaps are written out.
//   scores: one workgroup per (b, h, group): each active tile gets all 1024
//           dot products Qbar . Kbar in float32 from three bf16 MFMA products
//           of split operands, and its candidate entries are written in place.
//   select: one wavefront per (b, h, query block), the row's order-preserving
//           score keys in registers: the cut key is found bit by bit from the
//           top (32 passes of compares and ballot popcounts for static-ratio,
//           of fixed-point softmax-mass sums for dynamic-threshold); ties at
//           the cut go to the lower key index; the kept flags are compacted in
//           candidate (ascending) order. Rows longer than the register
//           capacity take a workgroup radix select (4 passes of 8 bits) with
//           the same keys, weights and tie rule.
#include "dr_internal.h"

namespace dr {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ inline float bf16_lo(unsigned int w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(unsigned int w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------------------
// Block mean pooling.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void pool_kernel(PoolParams p) {
  constexpr int LPR = D / 8;        // lanes per row (8 bf16 each)
  constexpr int RPI = 64 / LPR;     // rows per load instruction
  const int lane = threadIdx.x & 63;
  const long long g = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long long per = (long long)p.B * p.Hp * p.Sb;
  if (g >= 2 * per) return;
  const int which = (int)(g / per);
  const long long r = g - which * per;
  const int a = (int)(r % p.Sb);
  const int bh = (int)(r / p.Sb);
  const int b = bh / p.Hp, h = bh - b * p.Hp;
  const uint16_t* src = (which ? p.k : p.q) + ((size_t)(b * p.H + h) * p.S + (size_t)a * p.Bs) * D;
  const int n = min(p.Bs, p.S - a * p.Bs);
  const int col = (lane % LPR) * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int row = lane / LPR; row < n; row += RPI) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(src + (size_t)row * D + col);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16_lo(w[i]);
      acc[2 * i + 1] += bf16_hi(w[i]);
    }
  }
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += __shfl_xor(acc[i], off);
  if (lane < LPR) {
    float* dst = (which ? p.kbar : p.qbar) + ((size_t)(b * p.Hp + h) * p.Sb + a) * D + col;
    const float fn = (float)n;
    floatx4 lo = {acc[0] / fn, acc[1] / fn, acc[2] / fn, acc[3] / fn};
    floatx4 hi = {acc[4] / fn, acc[5] / fn, acc[6] / fn, acc[7] / fn};
    *reinterpret_cast<floatx4*>(dst) = lo;
    *reinterpret_cast<floatx4*>(dst + 4) = hi;
  }
}

// ---------------------------------------------------------------------------
// Candidate tiles. The candidate mask is the same for every (b, h), so the
// map from (query block, key block) to CSR position is built once per group
// of 32 consecutive query blocks: their candidate entries are one contiguous
// CSR range, turned into per-row bitmaps over the key blocks in LDS plus, per
// row and 32-block word, the CSR position of the word's first entry. A word
// with a bit set in any row is an active 32x32 tile; its bitmaps and
// positions are written out in tile order.
// ---------------------------------------------------------------------------
constexpr int kPrepThreads = 256;

__global__ __launch_bounds__(kPrepThreads) void tile_desc_kernel(ScoreParams p) {
  extern __shared__ unsigned int s_bits[];          // [32][nword] row bitmaps
  __shared__ int s_ntiles;
  const TileDesc& td = p.tiles;
  const int nword = td.nword;
  int* s_pos = reinterpret_cast<int*>(s_bits + 32 * nword);   // [32][nword]
  int* s_tiles = s_pos + 32 * nword;                          // active words
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = blockIdx.x, a0 = grp * 32;

  for (int i = tid; i < 32 * nword; i += kPrepThreads) s_bits[i] = 0;
  __syncthreads();
  for (int m = wave; m < 32; m += kPrepThreads / 64) {
    const int a = a0 + m;
    if (a >= p.Sb) continue;
    const int e1 = p.row_ptr[a + 1];
    // 8 column loads in flight per lane before their bits are set
    for (int e0 = p.row_ptr[a] + lane; e0 < e1; e0 += 8 * 64) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = e0 + 64 * u < e1 ? p.cols[e0 + 64 * u] : -1;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (c[u] >= 0) atomicOr(&s_bits[m * nword + (c[u] >> 5)], 1u << (c[u] & 31));
    }
  }
  __syncthreads();
  for (int m = wave; m < 32; m += kPrepThreads / 64) {
    const int a = a0 + m;
    int run = a < p.Sb ? p.row_ptr[a] : 0;
    for (int w0 = 0; w0 < nword; w0 += 64) {
      const int w = w0 + lane;
      const int cnt = w < nword ? __popc(s_bits[m * nword + w]) : 0;
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      if (w < nword) s_pos[m * nword + w] = run + incl - cnt;
      run += __shfl(incl, 63);
    }
  }
  if (wave == 0) {
    int n = 0;
    for (int w0 = 0; w0 < nword; w0 += 64) {
      const int w = w0 + lane;
      unsigned int any = 0;
      if (w < nword)
        for (int m = 0; m < 32; ++m) any |= s_bits[m * nword + w];
      const unsigned long long bal = __ballot(any != 0);
      const int before = __builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0));
      if (any) s_tiles[n + before] = w;
      n += __popcll(bal);
    }
    if (lane == 0) {
      s_ntiles = n;
      td.count[grp] = n;
    }
  }
  __syncthreads();
  const int ntiles = s_ntiles;
  const size_t base = (size_t)grp * nword;
  for (int j = tid; j < ntiles; j += kPrepThreads) td.word[base + j] = s_tiles[j];
  for (int i = tid; i < ntiles * 32; i += kPrepThreads) {
    const int j = i >> 5, m = i & 31, t = s_tiles[j];
    td.bits[(base + j) * 32 + m] = s_bits[m * nword + t];
    td.pos[(base + j) * 32 + m] = s_pos[m * nword + t];
  }
}

// ---------------------------------------------------------------------------
// Candidate scores: float32 dot products from the bf16 MFMA in three parts.
// A workgroup (4 wavefronts) owns one group of 32 query blocks of one (b, h);
// the waves share the group's active tiles, compute all 1024 dot products of
// a tile and write its candidate entries straight to their CSR positions (a
// popcount into the row's bitmap). The pooled K rows of a wave's next tile
// are loaded while the current one is on the matrix cores.
// Each float32 operand is split as x = hi + lo (bf16 each, exact up to
// 2^-17 |x|) and q.k is accumulated in float32 as ql.kh + qh.kl + qh.kh with
// v_mfma_f32_32x32x16_bf16 (the dropped ql.kl and the split remainders are
// below 2^-16 |q||k| per product): a third of the issue cycles of the float32
// MFMA for the same result to ~1e-6 at these score magnitudes.
// Operand layout (32x32x16): A lane l holds row l%32, dims 16*kk + 8*(l/32)
// + (0..7); B likewise for column l%32; D element i of lane l is (row
// 8*(i/4) + 4*(l/32) + i%4, column l%32).
// ---------------------------------------------------------------------------
constexpr int kScoreThreads = 256;

// x = hi + lo + r with hi = bf16(x), lo = bf16(x - hi) (both round to nearest
// even; x - hi is exact in float32) and |r| <= 2^-17 |x|.
__device__ inline void split(const floatx8& x, bf16x8& hi, bf16x8& lo) {
  hi = __builtin_convertvector(x, bf16x8);
  const floatx8 back = __builtin_convertvector(hi, floatx8);
  lo = __builtin_convertvector(x - back, bf16x8);
}

__device__ inline floatx8 load8(const float* src) {
  const floatx4 a = *reinterpret_cast<const floatx4*>(src);
  const floatx4 b = *reinterpret_cast<const floatx4*>(src + 4);
  return floatx8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

template <int D>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreParams p, const uint32_t* __restrict__ dbits,
                                                             const int32_t* __restrict__ dpos) {
  constexpr int KS = D / 16;   // 16-dim steps of v_mfma_f32_32x32x16_bf16
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const TileDesc& td = p.tiles;
  // (b, h) major: an XCD works through whole heads, whose pooled Q and K
  // (2 * S_b * D * 4 bytes) then stay in its L2
  const int w = xcd_contiguous(blockIdx.x, gridDim.x);
  const int bm = w / td.ngroups;          // b * Hm + hm
  const int grp = w - bm * td.ngroups, a0 = grp * 32;
  const int b = bm / p.Hm, hm = bm - b * p.Hm;
  const long long out_base = (long long)bm * p.nnz;
  const int ntiles = td.count[grp];
  const size_t dbase = (size_t)grp * td.nword;
  __shared__ int s_word[kMaxBlocks / 32];   // key tile of each active tile
  for (int i = threadIdx.x; i < ntiles; i += kScoreThreads) s_word[i] = td.word[dbase + i];
  __syncthreads();

  const int m32 = lane & 31, half = lane >> 5;
  const int row = a0 + m32;
  const bool row_ok = row < p.Sb;
  // pooled head index of head j of the score: per-head mode uses head hm,
  // fused mode sums heads 0..g-1
  auto pooled = [&](int j) -> size_t { return (size_t)(b * p.Hp + (p.g == 1 ? hm : j)) * p.Sb; };
  // this lane's 8 dims of 16-dim step kk: 16*kk + 8*half + (0..7), as hi + lo
  bf16x8 qh[KS], ql[KS];
  auto load_q = [&](int j) {
    const float* src = p.qbar + (pooled(j) + (row_ok ? row : 0)) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      floatx8 v = {0, 0, 0, 0, 0, 0, 0, 0};
      if (row_ok) v = load8(src + 16 * kk);
      split(v, qh[kk], ql[kk]);
    }
  };
  // K rows past S_b read the last row (every lane loads, so the loads are
  // unconditional and counted exactly) and are zeroed at use
  auto load_k = [&](floatx8* kv, int t, int hh) {
    const int kc = min(t * 32 + m32, p.Sb - 1);
    const float* ksrc = p.kbar + (pooled(hh) + kc) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) kv[kk] = load8(ksrc + 16 * kk);
  };
  auto mma = [&](floatx16& acc, const floatx8* kv, int t) {
    const bool kc_ok = t * 32 + m32 < p.Sb;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      bf16x8 kh, kl;
      split(kc_ok ? kv[kk] : floatx8{0, 0, 0, 0, 0, 0, 0, 0}, kh, kl);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ql[kk], kh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qh[kk], kl, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qh[kk], kh, acc, 0, 0, 0);
    }
  };
  // element i of this lane is (row 8*(i/4) + 4*half + i%4, key block t*32 + m32).
  // A tile's 32 bitmaps and positions are wave-uniform: scalar loads of both
  // halves' rows, selected per lane.
  struct Desc {
    unsigned int b[32];
    int ps[32];
  };
  auto load_desc = [&](Desc& dsc, int j) {
    const size_t at = (size_t)__builtin_amdgcn_readfirstlane((int)((dbase + j) * 32));
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      dsc.b[m] = dbits[at + m];
      dsc.ps[m] = dpos[at + m];
    }
  };
  auto store = [&](const floatx16& acc, const Desc& dsc) {
    const unsigned int below = (1u << m32) - 1u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m0 = 8 * (i >> 2) + (i & 3);
      const unsigned int bits = half ? dsc.b[m0 + 4] : dsc.b[m0];
      const int ps = half ? dsc.ps[m0 + 4] : dsc.ps[m0];
      if ((bits >> m32) & 1u) p.scores[out_base + ps + __popc(bits & below)] = acc[i] * p.scale;
    }
  };

  Desc dsc;
  if (p.g == 1) {
    // per tile: its bitmaps and positions are requested first, then the
    // products, then the next tile's K rows, so the stores wait only for the
    // former (loads complete in issue order)
    // The next tile's K rows are requested step by step as the current
    // tile's are split for the matrix cores, so they are in flight during
    // its products and stores; the last tile's rows are loaded once more
    // rather than branched around, so every iteration issues the same loads.
    load_q(0);
    floatx8 kv[KS];
    int j = wave;
    if (j < ntiles) {
      int t = s_word[j];
      load_k(kv, t, 0);
      while (true) {
        load_desc(dsc, j);
        __builtin_amdgcn_sched_barrier(0);
        const int jn = j + kScoreThreads / 64;
        const int tn = s_word[min(jn, ntiles - 1)];
        const float* knext = p.kbar + (pooled(0) + min(tn * 32 + m32, p.Sb - 1)) * D + 8 * half;
        const bool kc_ok = t * 32 + m32 < p.Sb;
        floatx16 acc = {};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          bf16x8 kh, kl;
          split(kc_ok ? kv[kk] : floatx8{0, 0, 0, 0, 0, 0, 0, 0}, kh, kl);
          kv[kk] = load8(knext + 16 * kk);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ql[kk], kh, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qh[kk], kl, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qh[kk], kh, acc, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        store(acc, dsc);
        if (jn >= ntiles) break;
        j = jn;
        t = tn;
      }
    }
  } else {
    for (int j = wave; j < ntiles; j += kScoreThreads / 64) {
      const int t = s_word[j];
      load_desc(dsc, j);
      floatx16 acc = {};
      for (int hh = 0; hh < p.g; ++hh) {
        load_q(hh);
        floatx8 kv[KS];
        load_k(kv, t, hh);
        mma(acc, kv, t);
      }
      store(acc, dsc);
    }
  }
}

// ---------------------------------------------------------------------------
// Selection.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 256;

__device__ inline unsigned int order_key(float s) {
  unsigned int u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0;  // -0 orders as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline float key_to_float(unsigned int k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Fixed-point (2^-32) weight of a score for the mass histograms:
// floor(exp(s - max) * 2^32), exact integer sums, order-independent.
__device__ inline unsigned long long mass_weight(float s, float smax) {
  const float e = __expf(s - smax);
  return (unsigned long long)(e * 4294967296.0f);
}

__device__ inline int static_keep(int n, double ratio) {
#pragma clang fp contract(off)
  const double x = ratio * (double)n - kCountGuard;
  int k = (int)ceil(x);
  if (k < 1) k = 1;
  if (k > n) k = n;
  return k;
}

// Histogram weight: counts (static-ratio) or fixed-point mass (dynamic).
template <bool DYN> struct Weight { typedef unsigned int type; };
template <> struct Weight<true> { typedef unsigned long long type; };

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectParams p) {
  extern __shared__ float s_sc[];
  __shared__ unsigned long long s_hist[256];
  __shared__ unsigned long long s_red[kSelThreads / 64];
  __shared__ float s_redf[kSelThreads / 64];
  __shared__ int s_wave[2][kSelThreads / 64];
  __shared__ unsigned long long s_pick[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int a = blockIdx.x;
  const int bm = blockIdx.y;             // b * Hm + hm
  const int r0 = p.row_ptr[a];
  const int n = p.row_ptr[a + 1] - r0;
  if (n <= p.min_n) return;
  const float* sc = p.scores + (long long)bm * p.nnz + r0;
  for (int i = tid; i < n; i += kSelThreads) s_sc[i] = sc[i];
  __syncthreads();

  const bool dyn = p.mode == 1;
  const bool keep_all = n == 0 || (dyn ? p.tau >= 1.0 : static_keep(n, p.ratio) >= n);
  unsigned int T = 0;
  unsigned long long tie_keep = 0;
  if (!keep_all) {
    float smax = -INFINITY;
    unsigned long long need;
    if (dyn) {
      float mx = -INFINITY;
      for (int i = tid; i < n; i += kSelThreads) mx = fmaxf(mx, s_sc[i]);
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      if (lane == 0) s_redf[wave] = mx;
      __syncthreads();
      smax = s_redf[0];
      for (int w = 1; w < kSelThreads / 64; ++w) smax = fmaxf(smax, s_redf[w]);
      unsigned long long z = 0;
      for (int i = tid; i < n; i += kSelThreads) z += mass_weight(s_sc[i], smax);
      for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
      if (lane == 0) s_red[wave] = z;
      __syncthreads();
      unsigned long long Z = 0;
      for (int w = 0; w < kSelThreads / 64; ++w) Z += s_red[w];
      need = (unsigned long long)ceil(p.tau * (double)Z);
    } else {
      need = (unsigned long long)static_keep(n, p.ratio);
    }
    // radix select, most significant digit first: find the key T at which the
    // weight of keys > T is < need and of keys >= T is >= need.
    unsigned int prefix = 0, pmask = 0;
    unsigned long long rem = need;
    for (int shift = 24; shift >= 0; shift -= 8) {
      s_hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kSelThreads) {
        const unsigned int key = order_key(s_sc[i]);
        if ((key & pmask) == prefix)
          atomicAdd(&s_hist[(key >> shift) & 255u], dyn ? mass_weight(s_sc[i], smax) : 1ull);
      }
      __syncthreads();
      if (wave == 0) {
        // lane l holds bins 255-4l .. 252-4l (descending)
        unsigned long long v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = s_hist[255 - 4 * lane - j];
        const unsigned long long mine = v[0] + v[1] + v[2] + v[3];
        unsigned long long incl = mine;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const unsigned long long o = __shfl_up(incl, off);
          if (lane >= off) incl += o;
        }
        const unsigned long long excl = incl - mine;
        if (excl < rem && incl >= rem) {
          unsigned long long c = excl;
          int d = 255 - 4 * lane;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (c + v[j] >= rem) { d = 255 - 4 * lane - j; break; }
            c += v[j];
          }
          s_pick[0] = (unsigned long long)d;
          s_pick[1] = c;
        }
      }
      __syncthreads();
      const unsigned int d = (unsigned int)s_pick[0];
      rem -= s_pick[1];
      prefix |= d << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    T = prefix;
    // ties at T: keep the lowest-index ones until the remaining need is met
    if (dyn) {
      const unsigned long long wT = mass_weight(key_to_float(T), smax);
      tie_keep = (rem + wT - 1) / wT;
    } else {
      tie_keep = rem;
    }
  }

  // ordered compaction of the kept flags (candidate order is ascending)
  const int H = p.H;
  const int b = bm / p.Hm, hm = bm - b * p.Hm;
  const int h_lo = p.Hm == 1 ? 0 : hm, h_hi = p.Hm == 1 ? H : hm + 1;
  int kept_base = 0;
  long long tie_base = 0;
  for (int i0 = 0; i0 < n; i0 += kSelThreads) {
    const int i = i0 + tid;
    bool keep = false, tie = false;
    if (i < n) {
      if (keep_all) {
        keep = true;
      } else {
        const unsigned int key = order_key(s_sc[i]);
        keep = key > T;
        tie = key == T;
      }
    }
    const unsigned long long mt = __ballot(tie);
    const int tie_before = __builtin_amdgcn_mbcnt_hi((unsigned)(mt >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)mt, 0));
    if (lane == 0) s_wave[0][wave] = __popcll(mt);
    __syncthreads();
    int toff = 0, ttot = 0;
    for (int w = 0; w < kSelThreads / 64; ++w) {
      toff += w < wave ? s_wave[0][w] : 0;
      ttot += s_wave[0][w];
    }
    if (tie && (unsigned long long)(tie_base + toff + tie_before) < tie_keep) keep = true;
    tie_base += ttot;
    const unsigned long long mk = __ballot(keep);
    const int k_before = __builtin_amdgcn_mbcnt_hi((unsigned)(mk >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)mk, 0));
    if (lane == 0) s_wave[1][wave] = __popcll(mk);
    __syncthreads();
    int koff = 0, ktot = 0;
    for (int w = 0; w < kSelThreads / 64; ++w) {
      koff += w < wave ? s_wave[1][w] : 0;
      ktot += s_wave[1][w];
    }
    if (keep) {
      const int col = p.cols[r0 + i];
      for (int h = h_lo; h < h_hi; ++h)
        p.kept_col[(long long)(b * H + h) * p.nnz + r0 + kept_base + koff + k_before] = col;
    }
    kept_base += ktot;
    __syncthreads();
  }
  if (tid == 0)
    for (int h = h_lo; h < h_hi; ++h) p.kept_cnt[(long long)(b * H + h) * p.Sb + a] = kept_base;
}


// One wavefront per row of at most 64 * NR candidates; candidate i of the
// row sits in slot i / 64 of lane i % 64 (slots are visited in runs of 8, and
// a run past the row's end is skipped). The radix select is that of the
// workgroup kernel (same keys, weights, digit order and tie rule, so the same
// cut), on a histogram of the wave's own in LDS: no workgroup barrier. LDS
// operations of one wavefront complete in issue order, so a lane reads the
// bins after every lane's additions have landed.
template <int NR, bool DYN>
__global__ __launch_bounds__(256) void select_wave_kernel(SelectParams p) {
  typedef typename Weight<DYN>::type W;
  static_assert(NR % 8 == 0, "slots come in runs of 8");
  __shared__ W s_hist[4][256];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int a = blockIdx.x * 4 + wv;
  if (a >= p.Sb) return;
  const int bm = blockIdx.y;             // b * Hm + hm
  const int r0 = p.row_ptr[a];
  const int n = p.row_ptr[a + 1] - r0;
  if (n > 64 * NR) return;               // left to the workgroup kernel
  const int ns = (n + 63) >> 6;          // slots in use
  const float* sc = p.scores + (long long)bm * p.nnz + r0;
  W* hist = s_hist[wv];

  const bool keep_all = n == 0 || (DYN ? p.tau >= 1.0 : static_keep(n, p.ratio) >= n);
  unsigned int key[NR];
  W wt[DYN ? NR : 1];
  unsigned int T = 0;
  unsigned long long tie_keep = 0;
  if (!keep_all) {
    unsigned int kmax = 0;
#pragma unroll
    for (int j = 0; j < NR; ++j) key[j] = 0;
#pragma unroll
    for (int r = 0; r < NR / 8; ++r) {
      if (8 * r >= ns) break;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int j = 8 * r + jj, i = j * 64 + lane;
        if (i < n) key[j] = order_key(sc[i]);
        kmax = max(kmax, key[j]);
      }
    }
    unsigned long long need;
    float smax = 0.0f;
    if (DYN) {
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) kmax = max(kmax, (unsigned int)__shfl_xor((int)kmax, off));
      smax = key_to_float(kmax);
      unsigned long long z = 0;
#pragma unroll
      for (int j = 0; j < NR; ++j) wt[DYN ? j : 0] = 0;
#pragma unroll
      for (int r = 0; r < NR / 8; ++r) {
        if (8 * r >= ns) break;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int j = 8 * r + jj;
          if (j * 64 + lane < n) wt[DYN ? j : 0] = mass_weight(key_to_float(key[j]), smax);
          z += wt[DYN ? j : 0];
        }
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
      need = (unsigned long long)ceil(p.tau * (double)z);
    } else {
      need = (unsigned long long)static_keep(n, p.ratio);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) hist[lane + 64 * x] = 0;
    // most significant digit first: T is the key at which the weight of keys
    // > T is < need and of keys >= T is >= need
    unsigned int prefix = 0, pmask = 0;
    unsigned long long rem = need;
    for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
      for (int r = 0; r < NR / 8; ++r) {
        if (8 * r >= ns) break;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int j = 8 * r + jj;
          if (j * 64 + lane < n && (key[j] & pmask) == prefix)
            atomicAdd(&hist[(key[j] >> shift) & 255u], DYN ? wt[DYN ? j : 0] : (W)1);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // lane l holds bins 255-4l .. 252-4l (descending), and clears them
      W v[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) v[x] = hist[255 - 4 * lane - x];
#pragma unroll
      for (int x = 0; x < 4; ++x) hist[255 - 4 * lane - x] = 0;
      const unsigned long long mine = (unsigned long long)v[0] + v[1] + v[2] + v[3];
      unsigned long long incl = mine;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned long long o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      const unsigned long long excl = incl - mine;
      // exactly one lane holds the bin at which the running weight reaches rem
      const bool here = excl < rem && incl >= rem;
      unsigned long long c = excl;
      int dg = 255 - 4 * lane;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        if (c + v[x] >= rem) { dg = 255 - 4 * lane - x; break; }
        c += v[x];
      }
      const int src = __builtin_ctzll(__ballot(here));
      const unsigned int d = (unsigned int)__shfl(dg, src);
      rem -= __shfl(c, src);
      prefix |= d << shift;
      pmask |= 255u << shift;
    }
    T = prefix;
    // ties at T: keep the lowest-index ones until the remaining need is met
    if (DYN) {
      const unsigned long long wT = mass_weight(key_to_float(T), smax);
      tie_keep = (rem + wT - 1) / wT;
    } else {
      tie_keep = rem;
    }
  }

  // ordered compaction of the kept flags (candidate order is ascending)
  const int H = p.H;
  const int b = bm / p.Hm, hm = bm - b * p.Hm;
  const int h_lo = p.Hm == 1 ? 0 : hm, h_hi = p.Hm == 1 ? H : hm + 1;
  int kept = 0;
  unsigned long long tie_base = 0;
#pragma unroll
  for (int r = 0; r < NR / 8; ++r) {
    if (8 * r >= ns) break;
    int col[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int i = (8 * r + jj) * 64 + lane;
      col[jj] = i < n ? p.cols[r0 + i] : 0;
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = 8 * r + jj, i = j * 64 + lane;
      const bool valid = i < n;
      bool keep = valid && (keep_all || key[j] > T);
      const bool tie = valid && !keep_all && key[j] == T;
      const unsigned long long mt = __ballot(tie);
      const int tie_before = __builtin_amdgcn_mbcnt_hi((unsigned)(mt >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)mt, 0));
      if (tie && tie_base + tie_before < tie_keep) keep = true;
      tie_base += __popcll(mt);
      const unsigned long long mk = __ballot(keep);
      const int k_before = __builtin_amdgcn_mbcnt_hi((unsigned)(mk >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)mk, 0));
      if (keep)
        for (int h = h_lo; h < h_hi; ++h) p.kept_col[(long long)(b * H + h) * p.nnz + r0 + kept + k_before] = col[jj];
      kept += __popcll(mk);
    }
  }
  if (lane == 0)
    for (int h = h_lo; h < h_hi; ++h) p.kept_cnt[(long long)(b * H + h) * p.Sb + a] = kept;
}
}  // namespace

hipError_t launch_pool(const PoolParams& p, hipStream_t stream) {
  const long long waves = 2LL * p.B * p.Hp * p.Sb;
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (p.D == 128)
    hipLaunchKernelGGL(pool_kernel<128>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(pool_kernel<64>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

size_t tile_desc_bytes(int Sb) {
  const size_t ng = (size_t)(Sb + 31) / 32, nword = ng;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al(ng * 4) + al(ng * nword * 4) + 2 * al(ng * nword * 32 * 4);
}

TileDesc tile_desc_at(void* base, int Sb) {
  const size_t ng = (size_t)(Sb + 31) / 32, nword = ng;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  unsigned char* c = static_cast<unsigned char*>(base);
  TileDesc t;
  t.count = reinterpret_cast<int32_t*>(c);
  c += al(ng * 4);
  t.word = reinterpret_cast<int32_t*>(c);
  c += al(ng * nword * 4);
  t.bits = reinterpret_cast<uint32_t*>(c);
  c += al(ng * nword * 32 * 4);
  t.pos = reinterpret_cast<int32_t*>(c);
  t.ngroups = (int)ng;
  t.nword = (int)nword;
  return t;
}

hipError_t launch_tile_desc(const ScoreParams& p, hipStream_t stream) {
  const int nword = p.tiles.nword;
  const size_t lds = (size_t)nword * (32 * 4 + 32 * 4 + 4);
  hipLaunchKernelGGL(tile_desc_kernel, dim3((unsigned)p.tiles.ngroups), dim3(kPrepThreads), lds, stream, p);
  return hipGetLastError();
}

hipError_t launch_scores(const ScoreParams& p, int B, hipStream_t stream) {
  const dim3 grid((unsigned)(p.tiles.ngroups * B * p.Hm));
  if (p.D == 128)
    hipLaunchKernelGGL(score_kernel<128>, grid, dim3(kScoreThreads), 0, stream, p, p.tiles.bits, p.tiles.pos);
  else
    hipLaunchKernelGGL(score_kernel<64>, grid, dim3(kScoreThreads), 0, stream, p, p.tiles.bits, p.tiles.pos);
  return hipGetLastError();
}

// Register capacity of the per-wave selection: 64 * kSelSlots candidates.
constexpr int kSelSlots = 40;

hipError_t launch_select(const SelectParams& p0, int B, hipStream_t stream) {
  SelectParams p = p0;
  p.min_n = 64 * kSelSlots;
  const dim3 wgrid((unsigned)((p.Sb + 3) / 4), (unsigned)(B * p.Hm));
  if (p.mode == 1)
    hipLaunchKernelGGL((select_wave_kernel<kSelSlots, true>), wgrid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((select_wave_kernel<kSelSlots, false>), wgrid, dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.max_row <= p.min_n) return e;
  const dim3 grid((unsigned)p.Sb, (unsigned)(B * p.Hm));
  hipLaunchKernelGGL(select_kernel, grid, dim3(kSelThreads), (size_t)p.max_row * sizeof(float), stream, p);
  return hipGetLastError();
}

}  // namespace dr
