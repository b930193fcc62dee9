// Block scoring and dual-mode selection on gfx950 ([DR] §3.2, block form;
// [DR] = "DynamicRad: Content-Adaptive Sparse Attention for Long Video
// Diffusion", arXiv 2604.20470).
//
//   pool:   one wavefront per (tensor, b, h, block): coalesced 16-byte bf16 loads
//           of the block's valid rows, float32 sums, cross-lane reduction, mean.
//           HBM-bound (reads Q and K once).
//   scores: one wavefront per (b, h, 32 query blocks): walks the 32 rows'
//           candidate lists in key-block order, and for every 32x32 tile of
//           (query block, key block) pairs that holds a candidate computes all
//           1024 dot products Qbar . Kbar with the fp32 MFMA (32x32x2), then
//           scatters the candidate entries into CSR order.
//   select: one workgroup per (b, h, query block): radix select (4 passes of
//           8 bits) over order-preserving score keys with integer histograms:
//           counts for static-ratio, fixed-point softmax mass for
//           dynamic-threshold; ties at the cut go to the lower key index; the
//           kept flags are compacted in candidate (ascending) order.
#include "dr_internal.h"

namespace dr {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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
// Candidate scores via fp32 MFMA tiles.
// v_mfma_f32_32x32x2_f32: A is 32x2 (lane l: row l%32, k = l/32), B is 2x32
// (lane l: column l%32, k = l/32), D is 32x32 (lane l: column l%32, element i:
// row 8*(i/4) + 4*(l/32) + i%4). The reduction dimension is split so that lane
// half h walks dims [h*D/2, (h+1)*D/2): each MFMA adds one dim from each half.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void score_kernel(ScoreParams p) {
  constexpr int HD = D / 2;
  __shared__ float tileT[32][33];
  const int lane = threadIdx.x;
  const int m = lane & 31, half = lane >> 5;
  const int a0 = blockIdx.x * 32;
  const int bm = blockIdx.y;              // b * Hm + hm
  const int b = bm / p.Hm, hm = bm - b * p.Hm;
  const int row = a0 + m;
  const bool row_ok = row < p.Sb;
  int cur = row_ok ? p.row_ptr[row] : 0;
  const int end = row_ok ? p.row_ptr[row + 1] : 0;
  const long long out_base = (long long)bm * p.nnz;
  // pooled head index of head j of the score: per-head mode uses head hm,
  // fused mode sums heads 0..g-1.
  auto pooled = [&](int j) -> size_t { return (size_t)(b * p.Hp + (p.g == 1 ? hm : j)) * p.Sb; };

  float qa[HD];
  if (p.g == 1) {
    const float* src = p.qbar + (pooled(0) + (row_ok ? row : 0)) * D + half * HD;
#pragma unroll
    for (int i = 0; i < HD; i += 4) {
      floatx4 v = row_ok ? *reinterpret_cast<const floatx4*>(src + i) : floatx4{0, 0, 0, 0};
      qa[i] = v[0]; qa[i + 1] = v[1]; qa[i + 2] = v[2]; qa[i + 3] = v[3];
    }
  }
  while (true) {
    // next key-block tile holding a candidate of any of the 32 rows
    int nxt = cur < end ? p.cols[cur] : 0x7fffffff;
    for (int off = 32; off > 0; off >>= 1) nxt = min(nxt, __shfl_xor(nxt, off));
    if (nxt == 0x7fffffff) break;
    const int c0 = nxt & ~31;
    const int kc = c0 + m;
    const bool kc_ok = kc < p.Sb;
    floatx16 acc = {};
    for (int j = 0; j < p.g; ++j) {
      if (p.g != 1) {
        const float* src = p.qbar + (pooled(j) + (row_ok ? row : 0)) * D + half * HD;
#pragma unroll
        for (int i = 0; i < HD; i += 4) {
          floatx4 v = row_ok ? *reinterpret_cast<const floatx4*>(src + i) : floatx4{0, 0, 0, 0};
          qa[i] = v[0]; qa[i + 1] = v[1]; qa[i + 2] = v[2]; qa[i + 3] = v[3];
        }
      }
      const float* ksrc = p.kbar + (pooled(j) + (kc_ok ? kc : 0)) * D + half * HD;
#pragma unroll
      for (int i = 0; i < HD; i += 4) {
        floatx4 kv = kc_ok ? *reinterpret_cast<const floatx4*>(ksrc + i) : floatx4{0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[i], kv[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[i + 1], kv[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[i + 2], kv[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[i + 3], kv[3], acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) tileT[8 * (i >> 2) + 4 * half + (i & 3)][m] = acc[i];
    __syncthreads();
    // scatter this tile's candidate entries of row m (both halves walk the
    // cursor; half 0 writes)
    while (cur < end) {
      const int c = p.cols[cur];
      if (c >= c0 + 32) break;
      if (half == 0) p.scores[out_base + cur] = tileT[m][c - c0] * p.scale;
      ++cur;
    }
    __syncthreads();
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

hipError_t launch_scores(const ScoreParams& p, int B, hipStream_t stream) {
  const dim3 grid((unsigned)((p.Sb + 31) / 32), (unsigned)(B * p.Hm));
  if (p.D == 128)
    hipLaunchKernelGGL(score_kernel<128>, grid, dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL(score_kernel<64>, grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_select(const SelectParams& p, int B, hipStream_t stream) {
  const dim3 grid((unsigned)p.Sb, (unsigned)(B * p.Hm));
  hipLaunchKernelGGL(select_kernel, grid, dim3(kSelThreads), (size_t)p.max_row * sizeof(float), stream, p);
  return hipGetLastError();
}

}  // namespace dr
