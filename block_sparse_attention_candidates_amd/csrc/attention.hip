// Flash-style forward attention on gfx950: block-sparse over kept KV blocks
// ([DR] §3.3 Eqs. 12-13 with eps -> 0) and dense (the App. A / Table 5
// baseline). [DR] = "DynamicRad: Content-Adaptive Sparse Attention for Long
// Video Diffusion", arXiv 2604.20470.
//
// Workgroup = 8 compute wavefronts + 4 loader wavefronts, 256 query rows of
// one (b, h). Each compute wavefront owns 32 query rows (one 32x32 MFMA tile);
// in sparse mode those rows are 256 / B_s query blocks. Sparse workgroups are
// remapped so that runs of 8 neighbouring query groups of a head execute
// together on one XCD, where the KV blocks their unions share hit in its L2.
//
// Setup (the only workgroup barriers): the kept lists of the workgroup's
// query blocks are ORed into per-block LDS bitmaps; their union is the set of
// KV blocks the workgroup streams, cut into 32-key units. The stream visits
// the union in round-robin order over the query blocks by rank in their kept
// lists (block c at key min over (slot s, rank i) of QB * i + s), so every
// compute wave meets its own blocks evenly along the stream and the waves,
// coupled through the ring, wait less for each other than in key order. The
// order is a function of the group's kept lists only: outputs are bitwise
// reproducible.
//
// Streaming without barriers: the loaders copy units from HBM/L2 straight into
// an LDS ring (6 or more slots) with direct-to-LDS loads (16 B per lane, no registers),
// each keeping one unit in flight, and publish a slot once its loads have
// landed. Each compute wavefront walks only the units of the KV blocks its own
// query block kept, announces its position, waits for the slot, computes. A
// loader refills a slot only after every compute wavefront has moved past the
// unit it held. Compute wavefronts therefore run out of phase with each other,
// and the two on a SIMD overlap one's MFMA with the other's softmax. Waits are
// bounded (a wave gives up after p.spin_limit polls, 2^26 by default; the
// protocol never needs that) and a wave that gives up sets a bit of
// g_attn_wait_flags, which the host reads back (take_wait_flags_attn).
//
// Per compute wavefront and 32-key unit (v_mfma_f32_32x32x16_bf16):
//   S^T = K Q^T : A = K rows read from LDS (16 B per lane), B = the wave's Q
//                 fragment in registers; lane l holds the 16 scores of query
//                 row l%32 for keys 8*(i/4) + 4*(l/32) + i%4.
//   softmax     : float32, exp2 with the scale folded into one FMA; the row max
//                 (three-input maxima) is shared by the two lane halves with
//                 one shuffle; the output is rescaled only when a row max grows
//                 by more than 2^8 (probabilities stay <= 256, exact after the
//                 final 1/l); padding keys get probability 0; the row sum adds
//                 the bf16 probabilities the PV product uses, two per
//                 v_dot2c_f32_bf16.
//   O^T += V^T P^T: B = the lane's own probabilities as bf16; A = V^T obtained
//                 from row-major V in LDS with the gfx950 transposing LDS read
//                 (ds_read_b64_tr_b16: a 16-lane group turns four 4-element
//                 row chunks into four 4-key columns), keys taken in the order
//                 in which each lane holds P.
// LDS rows are XOR-swizzled in 16-byte chunks (chosen per row so that the
// MFMA operand reads of a wave hit distinct banks); the loaders pick, per lane,
// the global chunk that belongs at each physical position.
#include "dr_internal.h"
#include "lds_dma.h"

namespace dr {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_v __attribute__((__vector_size__(4 * sizeof(__bf16))));
#define DR_LDS __attribute__((address_space(3)))

constexpr int kConsumers = 8;
// Four loaders with one unit in flight each publish every unit as soon as it
// lands and leave most of the ring to landed units; measured faster than
// three loaders with two in flight each (wan14b_720p static 12.1 -> 11.2 ms).
constexpr int kLoaders = 4;
constexpr int kThreads = (kConsumers + kLoaders) * 64;
constexpr int kRows = kConsumers * 32;       // query rows per workgroup
constexpr int kInflight = 1;                 // units in flight per loader
// Sparse work items per XCD run (see xcd_chunked): 8 measured best (wan14b_720p
// static 11.11 -> 10.78 ms, dynamic 38.8 -> 37.5 ms; 16: 10.88 / 37.96; 32:
// 11.65 / 40.9; one contiguous range per XCD was slower still)
constexpr int kXcdRun = 8;
constexpr int kMaxSlots = 16;                // ring depth limit, in 32-key units
constexpr int kLdsBytes = 160 * 1024;        // LDS per workgroup on gfx950
static_assert(kConsumers == 8, "the loaders read the 8 progress entries as two int4");
constexpr int kUnit = 32;
constexpr float kRescaleLog2 = 8.0f;         // rescale only past 2^8 growth
constexpr int kDone = 0x3fffffff;

template <int D, int NS>
struct Geo {
  static constexpr int RB = 2 * D;               // bytes per key row
  static constexpr int TBYTES = kUnit * RB;      // K (or V) bytes of a unit
  static constexpr int SLOT = 2 * TBYTES;        // K then V
  static constexpr int NLOAD = TBYTES / 1024;    // 1 KB direct loads per tensor
  static constexpr int RING = NS * SLOT;
  static_assert(NS >= kInflight * kLoaders + 1 && NS <= kMaxSlots, "ring depth");
};

// 16-byte chunk swizzles (physical chunk = logical chunk ^ swz(row)).
// K: the 16 lanes of a quarter-wave read 16 consecutive rows at one logical
// chunk; V: a half-wave's transposing reads cover 4 rows x 64 bytes.
template <int D>
__device__ inline int swz_k(int key) { return D == 128 ? (key & 15) : ((key >> 1) & 7); }
template <int D>
__device__ inline int swz_v(int key) { return D == 128 ? 4 * (key & 3) : 4 * ((key >> 1) & 1); }

__device__ inline int ld_relaxed(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ inline void st_relaxed(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ inline void compiler_fence() { asm volatile("" ::: "memory"); }

// max / sum of a value over the two 32-lane halves: v_permlane32_swap(v, v)
// yields the low half in both halves of one result and the high half in the other
__device__ inline float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Bits of the waits that gave up since the host last read them (kWaitAttn*).
__device__ unsigned int g_attn_wait_flags;

struct Shared {
  int prog[kConsumers];        // next unit each compute wave may read (16-byte aligned)
  int ready[kMaxSlots];        // unit index held by each slot (-1: none)
  int n_units;
  int tmax;                    // bound of the stream-order keys (setup)
  int pad[2];
};

template <int D, int BS, bool SPARSE, int NS>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnParams p) {
  using G = Geo<D, NS>;
  constexpr int kSlots = NS;
  constexpr int UPB = BS / kUnit;                 // units per KV block
  constexpr int QB = kRows / BS;                  // query blocks per workgroup
  constexpr int WPQ = BS / 32;                    // compute waves per query block
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* ring = smem;
  Shared* sh = reinterpret_cast<Shared*>(smem + G::RING);
  unsigned int* bits = reinterpret_cast<unsigned int*>(smem + G::RING + sizeof(Shared));

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // work item: (query group gx, head bh). Sparse: runs of kXcdRun neighbouring
  // groups, whose unions share most KV blocks, run together on one XCD (one L2)
  int gx = blockIdx.x, bh = blockIdx.y;
  if constexpr (SPARSE) {
    const int w = xcd_chunked(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y, kXcdRun);
    gx = w % gridDim.x;
    bh = w / gridDim.x;
  }
  const int row0 = gx * kRows;
  const size_t base = (size_t)bh * p.S * D;
  // query block of group slot s (sparse: per-(b, h) grouping mode)
  int gmode = 0;
  if constexpr (SPARSE) {
    if (p.group_mode) {
      gmode = p.group_mode[bh];
      if (gmode < 0 || gmode >= kGroupModes || group_count(p.grp, gmode) == 0) gmode = 0;
    }
    if (gx >= group_count(p.grp, gmode)) return;   // uniform: before any barrier
  }
  auto qblock = [&](int s) -> int {
    if constexpr (SPARSE) return group_block(p.grp, gmode, gx, s);
    else return row0 / BS + s;
  };
  const int nword = (p.Sb + 31) >> 5;
  unsigned int* uword = bits + QB * nword;        // union of the query blocks' key bitmaps
  int* wpre = reinterpret_cast<int*>(uword + nword);  // exclusive prefix popcounts
  uint16_t* stream = reinterpret_cast<uint16_t*>(wpre + nword);  // key block of each union step

  // ---------------- setup ----------------
  if (tid < kSlots) sh->ready[tid] = -1;
  if (tid < kConsumers) sh->prog[tid] = 0;
  if constexpr (SPARSE) {
    // kept list of group slot s, its length clamped to the candidate row
    auto kept_of = [&](int s, int& cnt) -> const int32_t* {
      const int qb = qblock(s);
      cnt = 0;
      if (qb < 0 || qb >= p.Sb) return nullptr;
      cnt = min(p.kept_cnt[(long long)bh * p.Sb + qb], p.row_ptr[qb + 1] - p.row_ptr[qb]);
      return p.kept_col + (long long)bh * p.nnz + p.row_ptr[qb];
    };
    // union step (position among the union's key blocks) of key block c
    auto union_index = [&](int c) -> int {
      return wpre[c >> 5] + __popc(uword[c >> 5] & ((1u << (c & 31)) - 1u));
    };
    for (int i = tid; i < QB * nword; i += kThreads) bits[i] = 0;
    if (tid == 0) sh->tmax = 0;
    __syncthreads();
    if (wave < QB) {
      int cnt;
      const int32_t* kl = kept_of(wave, cnt);
      for (int i = lane; i < cnt; i += 64) {
        const int c = kl[i];
        if (c >= 0 && c < p.Sb) atomicOr(&bits[wave * nword + (c >> 5)], 1u << (c & 31));
      }
      if (lane == 0) atomicMax(&sh->tmax, QB * cnt);
    }
    __syncthreads();
    for (int wi = tid; wi < nword; wi += kThreads) {
      unsigned int u = 0;
      for (int s = 0; s < QB; ++s) u |= bits[s * nword + wi];
      uword[wi] = u;
    }
    __syncthreads();
    // exclusive prefix popcounts of a bitmap (one wavefront); returns the total
    auto prefix = [&](const unsigned int* words, int* pre, int n) -> int {
      int run = 0;
      for (int w0 = 0; w0 < n; w0 += 64) {
        const int wi = w0 + lane;
        const int c = wi < n ? __popc(words[wi]) : 0;
        int incl = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int o = __shfl_up(incl, off);
          if (lane >= off) incl += o;
        }
        if (wi < n) pre[wi] = run + incl - c;
        run += __shfl(incl, 63);
      }
      return run;
    };
    if (wave == 0) {
      const int U = prefix(uword, wpre, nword);
      if (lane == 0) sh->n_units = U * UPB;
    }
    __syncthreads();
    // Stream order: the union's key blocks in round-robin order over the group
    // slots by rank in their kept lists. Block c gets the key t(c) = min over
    // the slots s keeping it at rank i of QB * i + s; steps ascend in t. Each
    // slot then meets its i-th kept block no later than round i of the stream,
    // so its work is spread evenly over the stream, whatever the key order of
    // its list. Setup scratch lives in the ring (unused until streaming).
    const int U = sh->n_units / UPB;
    const int T = sh->tmax;                        // keys lie in [0, T)
    const int tw = (T + 31) >> 5;
    unsigned int* tmin = reinterpret_cast<unsigned int*>(ring);      // [U] key of each union step
    unsigned int* tbit = tmin + U;                                    // [tw] keys in use
    int* tpre = reinterpret_cast<int*>(tbit + tw);                    // [tw] their prefix counts
    for (int i = tid; i < U; i += kThreads) tmin[i] = 0xffffffffu;
    for (int i = tid; i < tw; i += kThreads) tbit[i] = 0;
    __syncthreads();
    if (wave < QB) {
      int cnt;
      const int32_t* kl = kept_of(wave, cnt);
      for (int i = lane; i < cnt; i += 64) {
        const int c = kl[i];
        if (c >= 0 && c < p.Sb) atomicMin(&tmin[union_index(c)], (unsigned)(QB * i + wave));
      }
    }
    __syncthreads();
    for (int i = tid; i < U; i += kThreads) {
      const unsigned int t = tmin[i];
      atomicOr(&tbit[t >> 5], 1u << (t & 31));
    }
    for (int i = tid; i < QB * nword; i += kThreads) bits[i] = 0;   // become step bitmaps
    __syncthreads();
    if (wave == 0) prefix(tbit, tpre, tw);
    __syncthreads();
    auto step_of = [&](unsigned int t) -> int { return tpre[t >> 5] + __popc(tbit[t >> 5] & ((1u << (t & 31)) - 1u)); };
    for (int wi = tid; wi < nword; wi += kThreads) {
      unsigned int m = uword[wi];
      int ui = wpre[wi];
      while (m) {
        const int b = __ffs(m) - 1;
        m &= m - 1;
        stream[step_of(tmin[ui++])] = (uint16_t)(wi * 32 + b);
      }
    }
    if (wave < QB) {
      int cnt;
      const int32_t* kl = kept_of(wave, cnt);
      for (int i = lane; i < cnt; i += 64) {
        const int c = kl[i];
        if (c >= 0 && c < p.Sb) {
          const int j = step_of(tmin[union_index(c)]);
          atomicOr(&bits[wave * nword + (j >> 5)], 1u << (j & 31));
        }
      }
    }
  } else {
    if (tid == 0) sh->n_units = (p.S + kUnit - 1) / kUnit;
  }
  __syncthreads();
  const int n_units = sh->n_units;

  if (wave >= kConsumers) {
    // ---------------- loader wavefronts ----------------
    const int L = wave - kConsumers;
    const uint16_t* __restrict__ Kg = p.k + base;
    const uint16_t* __restrict__ Vg = p.v + base;
    // key block of union step j
    auto block_of_step = [&](int j) -> int {
      if constexpr (!SPARSE) return j;
      else return (int)stream[j];
    };
    auto publish = [&](int u) {
      compiler_fence();
      st_relaxed(&sh->ready[u % kSlots], u);
    };
    // Byte offset of this lane's 16-byte chunk within a unit's K or V tile for
    // DMA instruction n: n * 1024 + dma_k[n % KM] (K) or + dma_v (V). The
    // swizzles depend on the row only through row mod (4 * KM) (K) or row mod 4
    // (V), so a few per-lane constants cover every instruction.
    constexpr int KM = D == 128 ? 4 : 2;
    auto lane_chunk = [&](int n, bool is_k) -> int {
      const int off = n * 1024 + 16 * lane;
      const int row = off / G::RB;
      const int pc = (off % G::RB) >> 4;
      const int lc = pc ^ (is_k ? swz_k<D>(row) : swz_v<D>(row));
      return row * G::RB + lc * 16 - n * 1024;
    };
    int dma_k[KM];
#pragma unroll
    for (int m = 0; m < KM; ++m) dma_k[m] = lane_chunk(m, true);
    const int dma_v = lane_chunk(0, false);
    auto issue = [&](int u) {
      const int j = u / UPB, q = u - j * UPB;
      const int key0 = uniform(block_of_step(j) * BS + q * kUnit);
      unsigned char* slot = ring + (u % kSlots) * G::SLOT;
      if (key0 + kUnit <= p.S) {
        const unsigned char* kb = reinterpret_cast<const unsigned char*>(Kg + (size_t)key0 * D);
        const unsigned char* vb = reinterpret_cast<const unsigned char*>(Vg + (size_t)key0 * D);
#pragma unroll
        for (int n = 0; n < G::NLOAD; ++n) dma16_s(kb + n * 1024, (unsigned)dma_k[n % KM], slot + n * 1024);
#pragma unroll
        for (int n = 0; n < G::NLOAD; ++n) dma16_s(vb + n * 1024, (unsigned)dma_v, slot + G::TBYTES + n * 1024);
        return;
      }
      // the tile running past the sequence end: rows clamped to the last token
#pragma unroll 1
      for (int t = 0; t < 2; ++t) {
        const uint16_t* src = t == 0 ? Kg : Vg;
#pragma unroll 1
        for (int n = 0; n < G::NLOAD; ++n) {
          const int off = n * 1024 + 16 * lane;
          const int row = off / G::RB;
          const int pc = (off % G::RB) >> 4;
          const int lc = pc ^ (t == 0 ? swz_k<D>(row) : swz_v<D>(row));
          const int key = min(key0 + row, p.S - 1);
          const uint16_t* g = src + (size_t)key * D + lc * 8;
          dma16(g, slot + t * G::TBYTES + n * 1024);
        }
      }
    };
    int k = 0;
    bool gave_up = false;
    for (int u = L; u < n_units; u += kLoaders, ++k) {
      if (k >= kInflight) {
        wait_vmcnt<2 * G::NLOAD * (kInflight - 1)>();
        publish(u - kLoaders * kInflight);
      }
      // The slot's previous unit (u - kSlots) must be passed by every compute
      // wave and must itself have been published: a unit that no wave needs
      // can otherwise still be landing when the slot is refetched.
      int spins = 0;
      while (true) {
        // explicit LDS loads: a generic (flat) load would also wait for this
        // wave's copies in flight
        const volatile DR_LDS intx4* pv = (const volatile DR_LDS intx4*)(&sh->prog[0]);
        const intx4 a = pv[0];
        const intx4 b = pv[1];
        const int mn = uniform(min(min(min(a[0], a[1]), min(a[2], a[3])), min(min(b[0], b[1]), min(b[2], b[3]))));
        const bool free_slot = mn >= u - kSlots + 1 &&
                               (u < kSlots || uniform(ld_relaxed(&sh->ready[u % kSlots])) == u - kSlots);
        if (free_slot) break;
        if (++spins > p.spin_limit) {
          gave_up = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      compiler_fence();
      // raised wave priority while issuing: the copies of a unit leave in
      // one burst instead of interleaving with the compute waves' issue
      __builtin_amdgcn_s_setprio(2);
      issue(u);
      __builtin_amdgcn_s_setprio(0);
    }
    wait_vmcnt<0>();
    const int first = max(L, L + kLoaders * (k - kInflight));
    for (int u = first; u < n_units; u += kLoaders) publish(u);
    if (gave_up && lane == 0) atomicOr(&g_attn_wait_flags, kWaitAttnLoader);
    return;
  }

  // ---------------- compute wavefronts ----------------
  const int half = lane >> 5, l32 = lane & 31;
  int wrow0 = row0 + wave * 32;
  if constexpr (SPARSE) {
    const int qb = qblock(wave / WPQ);
    wrow0 = qb >= 0 ? qb * BS + (wave % WPQ) * 32 : p.S;
  }
  bf16x8 qf[D / 16];
  {
    const int r = wrow0 + l32;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 w = {0, 0, 0, 0};
      if (r < p.S) w = *reinterpret_cast<const u32x4*>(p.q + base + (size_t)r * D + kk * 16 + half * 8);
      qf[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }
  floatx16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = floatx16{};
  const bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
  const float c = p.scale_log2;
  const bool c_pos = c >= 0.f;
  const float c_abs = fabsf(c);
  float m_ref = -INFINITY;   // reference row max of s * c (log2 units)
  float l_run = 0.f;

  // A = V^T operands for one 32-dim tile: lane l takes dims dt*32 + l%32 and,
  // for MFMA step j, keys 16j + 8r + 4*half + (0..3) from transposing read r.
  auto load_v = [&](const unsigned char* sv, int dt, bf16x8 (&va)[2]) {
    const int kq = (lane & 15) >> 2;
    const int dim = dt * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bf16x4_v part[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int key = 16 * j + 8 * r + 4 * half + kq;
        const int ch = (dim >> 3) ^ swz_v<D>(key);
        part[r] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((DR_LDS bf16x4_v*)(sv + key * G::RB + ch * 16 + (dim & 7) * 2));
      }
      va[j] = bf16x8{part[0][0], part[0][1], part[0][2], part[0][3], part[1][0], part[1][1], part[1][2], part[1][3]};
    }
  };

  auto compute = [&](const unsigned char* slot, int key0) {
    const unsigned char* sk = slot;
    const unsigned char* sv = slot + G::TBYTES;
    floatx16 s = {};
#pragma unroll
    for (int k0 = 0; k0 < D / 16; k0 += 4) {
      bf16x8 ka[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ch = (2 * (k0 + kk) + half) ^ swz_k<D>(l32);
        ka[kk] = *reinterpret_cast<const bf16x8*>(sk + l32 * G::RB + ch * 16);
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], qf[k0 + kk], s, 0, 0, 0);
    }
    // the first V^T operands load while the softmax runs
    bf16x8 va[2][2];
    load_v(sv, 0, va[0]);
    // row max of s * c over the valid keys: |c| * max(s) for c >= 0, |c| * max(-s)
    // otherwise; padding keys (beyond S) are left out of the max and get p = 0
    const bool ragged = key0 + kUnit > p.S;
    float mx;
    if (c_pos && !ragged) {
      // three-input maxima: 16 values in 8 instructions
      const float m0 = fmaxf(fmaxf(s[0], s[1]), s[2]), m1 = fmaxf(fmaxf(s[3], s[4]), s[5]);
      const float m2 = fmaxf(fmaxf(s[6], s[7]), s[8]), m3 = fmaxf(fmaxf(s[9], s[10]), s[11]);
      const float m4 = fmaxf(fmaxf(s[12], s[13]), s[14]);
      mx = fmaxf(fmaxf(fmaxf(m0, m1), m2), fmaxf(fmaxf(m3, m4), s[15]));
    } else {
      // element i holds key key0 + 4*half + 8*(i/4) + i%4: valid iff below lim
      const int lim = p.S - key0 - 4 * half;
      mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool valid = 8 * (i >> 2) + (i & 3) < lim;
        mx = fmaxf(mx, valid ? (c_pos ? s[i] : -s[i]) : -INFINITY);
      }
    }
    mx = max_halves(mx) * c_abs;
    if (__ballot(mx - m_ref > kRescaleLog2) != 0ull) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
    }
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -m_ref));
    if (ragged) {
      const int lim = p.S - key0 - 4 * half;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + (i & 3) >= lim) x[i] = 0.f;
    }
    bf16x8 pb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const floatx8 f = {x[8 * j], x[8 * j + 1], x[8 * j + 2], x[8 * j + 3],
                         x[8 * j + 4], x[8 * j + 5], x[8 * j + 6], x[8 * j + 7]};
      pb[j] = __builtin_convertvector(f, bf16x8);
    }
    // row sum of the probabilities as the PV product uses them (bf16), two per
    // v_dot2c_f32_bf16 with float32 accumulation
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x2 pair = {pb[j][2 * i], pb[j][2 * i + 1]};
        l_run = __builtin_amdgcn_fdot2_f32_bf16(pair, kOnes2, l_run, false);
      }
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      if (dt + 1 < D / 32) load_v(sv, dt + 1, va[(dt + 1) & 1]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt & 1][j], pb[j], oacc[dt], 0, 0, 0);
    }
  };

  bool gave_up = false;
  auto consume = [&](int u, int key0) {
    compiler_fence();
    st_relaxed(&sh->prog[wave], u);
    int spins = 0;
    while (ld_relaxed(&sh->ready[u % kSlots]) != u) {
      if (++spins > p.spin_limit) {
        gave_up = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    compiler_fence();
    compute(ring + (u % kSlots) * G::SLOT, key0);
  };

  if (wrow0 < p.S) {
    if constexpr (SPARSE) {
      // this query block's union steps, in stream order
      const unsigned int* mine = bits + (wave / WPQ) * nword;
      for (int wi = 0; wi < nword; ++wi) {
        // wave-uniform words: the walk runs on the scalar unit
        unsigned int m = (unsigned)uniform((int)mine[wi]);
        while (m) {
          const int b = __ffs(m) - 1;
          m &= m - 1;
          const int j = wi * 32 + b;
          const int cblk = uniform((int)stream[j]);
#pragma unroll
          for (int q = 0; q < UPB; ++q) {
            const int key0 = cblk * BS + q * kUnit;
            if (key0 >= p.S) break;
            consume(j * UPB + q, key0);
          }
        }
      }
    } else {
      for (int u = 0; u < n_units; ++u) consume(u, u * kUnit);
    }
  }
  compiler_fence();
  st_relaxed(&sh->prog[wave], kDone);
  if (gave_up && lane == 0) atomicOr(&g_attn_wait_flags, kWaitAttnCompute);

  // ---------------- epilogue ----------------
  const float l_tot = sum_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int r = wrow0 + l32;
  if (r < p.S) {
    uint16_t* orow = p.o + base + (size_t)r * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const floatx4 f = {oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv, oacc[dt][4 * g + 2] * inv,
                           oacc[dt][4 * g + 3] * inv};
        const bf16x4 hb = __builtin_convertvector(f, bf16x4);
        *reinterpret_cast<u32x2*>(orow + dt * 32 + 8 * g + 4 * half) = __builtin_bit_cast(u32x2, hb);
      }
    }
  }
}

template <int D, int BS, bool SPARSE, int NS>
size_t lds_bytes(const AttnParams& p) {
  size_t lds = Geo<D, NS>::RING + sizeof(Shared);
  if (SPARSE) {
    const int nword = (p.Sb + 31) / 32;
    lds += (size_t)(kRows / BS) * nword * 4 + (size_t)nword * 8 + (((size_t)p.Sb * 2 + 15) & ~(size_t)15);
  }
  return lds;
}

// Ring depth: 9 slots of 32 keys at D = 128 (16 at D = 64) when the sparse
// bitmaps and stream table leave room for them, else 6 (12). The shallow ring
// also holds the setup scratch of the largest layouts (S_b = 16384: 64 KB of
// step keys and 32 KB of key bitmaps).
template <int D, int BS, bool SPARSE>
hipError_t launch_one(const AttnParams& p, hipStream_t stream) {
  constexpr int DEEP = D == 128 ? 9 : 16;
  constexpr int SHALLOW = D == 128 ? 6 : 12;
  // sparse: the widest grouping in use; a workgroup past its mode's group
  // count exits at once
  int gx = p.n_tiles;
  if (SPARSE && p.group_mode)
    for (int m = 1; m < kGroupModes; ++m) gx = max(gx, group_count(p.grp, m));
  const dim3 grid((unsigned)gx, (unsigned)p.BH);
  const size_t deep = lds_bytes<D, BS, SPARSE, DEEP>(p);
  const size_t shallow = lds_bytes<D, BS, SPARSE, SHALLOW>(p);
  if (deep <= (size_t)kLdsBytes)
    hipLaunchKernelGGL((attn_kernel<D, BS, SPARSE, DEEP>), grid, dim3(kThreads), deep, stream, p);
  else if (shallow <= (size_t)kLdsBytes)
    hipLaunchKernelGGL((attn_kernel<D, BS, SPARSE, SHALLOW>), grid, dim3(kThreads), shallow, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_attn(const AttnParams& p, int D, int Bs, hipStream_t stream) {
  if (D == 128 && Bs == 32) return launch_one<128, 32, true>(p, stream);
  if (D == 128 && Bs == 64) return launch_one<128, 64, true>(p, stream);
  if (D == 64 && Bs == 32) return launch_one<64, 32, true>(p, stream);
  if (D == 64 && Bs == 64) return launch_one<64, 64, true>(p, stream);
  if (D == 128 && Bs == 128) return launch_one<128, 128, true>(p, stream);
  if (D == 64 && Bs == 128) return launch_one<64, 128, true>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t take_wait_flags_attn(unsigned* flags, hipStream_t stream) {
  unsigned v = 0;
  hipError_t e = hipMemcpyFromSymbolAsync(&v, HIP_SYMBOL(g_attn_wait_flags), sizeof v, 0, hipMemcpyDeviceToHost,
                                          stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e == hipSuccess && v != 0) {
    static const unsigned zero = 0;
    e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_attn_wait_flags), &zero, sizeof zero, 0, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
  }
  *flags = v;
  return e;
}

hipError_t launch_dense_attn(const AttnParams& p, int D, hipStream_t stream) {
  if (D == 128) return launch_one<128, 32, false>(p, stream);
  if (D == 64) return launch_one<64, 32, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace dr
