// Flash-style forward attention on gfx950: block-sparse over kept KV blocks
// ([DR] §3.3 Eqs. 12-13 with eps -> 0) and dense (the App. A / Table 5
// baseline). [DR] = "DynamicRad: Content-Adaptive Sparse Attention for Long
// Video Diffusion", arXiv 2604.20470.
//
// Work decomposition. A workgroup of 8 wavefronts owns 256 consecutive query
// rows of one (b, h); each wavefront owns 32 rows (one 32x32 MFMA tile). In
// sparse mode those rows are 256 / B_s query blocks; the workgroup ORs their
// kept lists into LDS bitmaps and compacts the union of kept KV blocks, then
// streams that union through a double-buffered LDS stage: every KV block is
// fetched from HBM/L2 once per workgroup and used by each wavefront whose
// query block kept it (a wave-uniform bit test). Dense mode streams every
// 64-key block.
//
// Per wavefront and 32-key unit (CDNA4 v_mfma_f32_32x32x16_bf16):
//   S^T = K Q^T  : A = K rows from LDS (16 B per lane), B = the wavefront's Q
//                  fragment held in registers; lane l ends with the 16 scores of
//                  query row l%32 for keys 8*(i/4) + 4*(l/32) + i%4.
//   online softmax in float32 on those registers (exp2 with the scale folded
//                  into log2(e)); the two lane halves of a row exchange their
//                  maxima once (shuffle by 32).
//   O^T += V^T P^T: B = the lane's own probabilities packed to bf16; A = V^T
//                  read from LDS, where V was stored transposed with its keys
//                  permuted to match the order in which each lane holds P.
// KV loads are issued P steps ahead into registers (a ring unrolled at compile
// time), written to LDS one step ahead, one barrier per step.
#include "dr_internal.h"

namespace dr {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kRowsPerWG = 256;

// slot of key j (0..31) within its 32-key unit in the transposed V stage:
// slot 16*jj + 8*h + e holds key 16*jj + 8*(e/4) + 4*h + e%4.
__device__ __host__ constexpr int v_slot(int j) {
  return 16 * (j / 16) + 8 * ((j % 8) / 4) + 4 * ((j % 16) / 8) + (j % 4);
}

template <int D, int BS>
struct Stage {
  static constexpr int KSTR = D + 8;                 // bf16 per K row in LDS
  static constexpr int VSTR = BS + 8;                // bf16 per V^T row in LDS
  static constexpr int K_ELEMS = BS * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
  static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
  static constexpr int CHUNKS = BS * D / 8;          // 16-byte chunks per tensor
  static constexpr int CPT = CHUNKS >= kThreads ? CHUNKS / kThreads : 1;
  static constexpr int PREFETCH = CPT == 1 ? 4 : 2;  // steps in flight
  static constexpr size_t BYTES = 2 * (size_t)BUF_ELEMS * 2;
};

template <int D, int BS, bool SPARSE>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnParams p) {
  using St = Stage<D, BS>;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* stage = reinterpret_cast<uint16_t*>(smem);
  constexpr int NUNIT = BS / 32;
  constexpr int QB_PER_WG = kRowsPerWG / BS;           // query blocks per workgroup
  constexpr int WAVES_PER_QB = BS / 32;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int bh = blockIdx.y;
  const int tile = blockIdx.x;
  const int row0 = tile * kRowsPerWG;
  const int wrow0 = row0 + wave * 32;
  const size_t base = (size_t)bh * p.S * D;
  const uint16_t* __restrict__ Kg = p.k + base;
  const uint16_t* __restrict__ Vg = p.v + base;

  // ---- Q fragment (B operand of S^T = K Q^T) ----
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

  // ---- the KV block sequence ----
  int n_steps;
  const int* ulist = nullptr;
  const unsigned int* my_bits = nullptr;
  if constexpr (SPARSE) {
    const int nword = (p.Sb + 31) >> 5;
    unsigned int* bits = reinterpret_cast<unsigned int*>(smem + St::BYTES);
    int* list = reinterpret_cast<int*>(bits + QB_PER_WG * nword);
    __shared__ int s_cnt[kThreads / 64];
    for (int i = tid; i < QB_PER_WG * nword; i += kThreads) bits[i] = 0;
    __syncthreads();
    {
      const int slot = wave / WAVES_PER_QB;
      const int qb = row0 / BS + slot;
      if (wave % WAVES_PER_QB == 0 && qb < p.Sb) {
        const int32_t* kl = p.kept_col + (long long)bh * p.nnz + p.row_ptr[qb];
        const int cnt = p.kept_cnt[(long long)bh * p.Sb + qb];
        for (int i = lane; i < cnt; i += 64) {
          const int c = kl[i];
          if (c >= 0 && c < p.Sb) atomicOr(&bits[slot * nword + (c >> 5)], 1u << (c & 31));
        }
      }
    }
    __syncthreads();
    // compact the union in ascending order
    int total = 0;
    for (int w0 = 0; w0 < nword; w0 += kThreads) {
      const int wi = w0 + tid;
      unsigned int u = 0;
      if (wi < nword)
        for (int s = 0; s < QB_PER_WG; ++s) u |= bits[s * nword + wi];
      const int c = __popc(u);
      int incl = c;
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      if (lane == 63) s_cnt[wave] = incl;
      __syncthreads();
      int woff = 0, wtot = 0;
      for (int w = 0; w < kThreads / 64; ++w) {
        woff += w < wave ? s_cnt[w] : 0;
        wtot += s_cnt[w];
      }
      int pos = total + woff + incl - c;
      while (u) {
        const int bit = __ffs(u) - 1;
        list[pos++] = wi * 32 + bit;
        u &= u - 1;
      }
      total += wtot;
      __syncthreads();
    }
    n_steps = total;
    ulist = list;
    my_bits = bits + (wave / WAVES_PER_QB) * nword;
  } else {
    n_steps = (p.S + BS - 1) / BS;
  }

  const bool wave_rows = wrow0 < p.S;

  // ---- loads: ring of PREFETCH register stages ----
  u32x4 kr[St::PREFETCH][St::CPT], vr[St::PREFETCH][St::CPT];
  auto issue = [&](int ps, int j) {
    const int c = SPARSE ? ulist[j] : j;
#pragma unroll
    for (int i = 0; i < St::CPT; ++i) {
      const int ci = tid + i * kThreads;
      const int key = c * BS + ci / (D / 8);
      const int d0 = (ci % (D / 8)) * 8;
      u32x4 kw = {0, 0, 0, 0}, vw = {0, 0, 0, 0};
      if (ci < St::CHUNKS && key < p.S) {
        kw = *reinterpret_cast<const u32x4*>(Kg + (size_t)key * D + d0);
        vw = *reinterpret_cast<const u32x4*>(Vg + (size_t)key * D + d0);
      }
      kr[ps][i] = kw;
      vr[ps][i] = vw;
    }
  };
  auto store = [&](int ps, int buf) {
    uint16_t* sk = stage + buf * St::BUF_ELEMS;
    uint16_t* sv = sk + St::K_ELEMS;
#pragma unroll
    for (int i = 0; i < St::CPT; ++i) {
      const int ci = tid + i * kThreads;
      if (ci < St::CHUNKS) {
        const int kl = ci / (D / 8);
        const int d0 = (ci % (D / 8)) * 8;
        *reinterpret_cast<u32x4*>(sk + kl * St::KSTR + d0) = kr[ps][i];
        const int slot = (kl & ~31) + v_slot(kl & 31);
        const u32x4 w = vr[ps][i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sv[(d0 + 2 * e) * St::VSTR + slot] = (uint16_t)(w[e] & 0xffffu);
          sv[(d0 + 2 * e + 1) * St::VSTR + slot] = (uint16_t)(w[e] >> 16);
        }
      }
    }
  };

  floatx16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = floatx16{};
  float m_run = -INFINITY, l_run = 0.f;

  auto compute = [&](int buf, int c) {
    const uint16_t* sk = stage + buf * St::BUF_ELEMS;
    const uint16_t* sv = sk + St::K_ELEMS;
#pragma unroll
    for (int u = 0; u < NUNIT; ++u) {
      const int key0 = c * BS + u * 32;
      if (key0 >= p.S) break;
      floatx16 s = {};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(sk + (u * 32 + l32) * St::KSTR + kk * 16 + half * 8);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s, 0, 0, 0);
      }
      float x[16];
      float mloc = -INFINITY;
      const bool ragged = key0 + 32 > p.S;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        x[i] = s[i] * p.scale_log2;
        if (ragged && key0 + 8 * (i >> 2) + 4 * half + (i & 3) >= p.S) x[i] = -INFINITY;
        mloc = fmaxf(mloc, x[i]);
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        x[i] = __builtin_amdgcn_exp2f(x[i] - m_new);
        psum += x[i];
      }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
      bf16x8 pb[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        floatx8 f = {x[8 * j], x[8 * j + 1], x[8 * j + 2], x[8 * j + 3],
                     x[8 * j + 4], x[8 * j + 5], x[8 * j + 6], x[8 * j + 7]};
        pb[j] = __builtin_convertvector(f, bf16x8);
      }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sv + (dt * 32 + l32) * St::VSTR + u * 32 + 16 * j + 8 * half);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[j], oacc[dt], 0, 0, 0);
        }
      }
    }
  };

  // ---- main loop ----
#pragma unroll
  for (int ps = 0; ps < St::PREFETCH; ++ps)
    if (ps < n_steps) issue(ps, ps);
  for (int j0 = 0; j0 < n_steps; j0 += St::PREFETCH) {
#pragma unroll
    for (int ps = 0; ps < St::PREFETCH; ++ps) {
      const int j = j0 + ps;
      if (j >= n_steps) break;
      const int buf = j & 1;
      store(ps, buf);
      __syncthreads();
      if (j + St::PREFETCH < n_steps) issue(ps, j + St::PREFETCH);
      bool need = wave_rows;
      int c = j;
      if constexpr (SPARSE) {
        c = ulist[j];
        need = need && ((my_bits[c >> 5] >> (c & 31)) & 1u);
      }
      if (need) compute(buf, c);
    }
  }

  // ---- epilogue: normalise and store bf16 ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int r = wrow0 + l32;
  if (r < p.S) {
    uint16_t* orow = p.o + base + (size_t)r * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        floatx4 f = {oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv, oacc[dt][4 * g + 2] * inv,
                     oacc[dt][4 * g + 3] * inv};
        const bf16x4 hb = __builtin_convertvector(f, bf16x4);
        *reinterpret_cast<u32x2*>(orow + dt * 32 + 8 * g + 4 * half) = __builtin_bit_cast(u32x2, hb);
      }
    }
  }
}

template <int D, int BS, bool SPARSE>
hipError_t launch_one(const AttnParams& p, hipStream_t stream) {
  using St = Stage<D, BS>;
  size_t lds = St::BYTES;
  if (SPARSE) {
    const int nword = (p.Sb + 31) / 32;
    lds += (size_t)(kRowsPerWG / BS) * nword * 4 + (size_t)p.Sb * 4;
  }
  const dim3 grid((unsigned)p.n_tiles, (unsigned)p.BH);
  hipLaunchKernelGGL((attn_kernel<D, BS, SPARSE>), grid, dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_attn(const AttnParams& p, int D, int Bs, hipStream_t stream) {
  if (D == 128 && Bs == 32) return launch_one<128, 32, true>(p, stream);
  if (D == 128 && Bs == 64) return launch_one<128, 64, true>(p, stream);
  if (D == 64 && Bs == 32) return launch_one<64, 32, true>(p, stream);
  if (D == 64 && Bs == 64) return launch_one<64, 64, true>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_dense_attn(const AttnParams& p, int D, hipStream_t stream) {
  if (D == 128) return launch_one<128, 64, false>(p, stream);
  if (D == 64) return launch_one<64, 64, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace dr
