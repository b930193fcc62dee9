// Decay-state static-ratio selection on gfx950 ([DR] §3.2 "Static-ratio
// mode", Eq. 8, Algorithm 1; aggregation by "Density control within blocks",
// §3.1). [DR] = "DynamicRad: Content-Adaptive Sparse Attention for Long Video
// Diffusion", arXiv 2604.20470.
//
// The mask depends only on the layout, the radial configuration, (rho_1,
// rho_2) and the seed: it is built once and cached by the caller. For every
// frame pair (i, j), t = |i - j|, that is retained (t mod sf(t) = 0):
//   t <= 1   all pairs of P(i, j) are selected (rho = 1; t = 0 is dense);
//   t >  1   k = max(1, floor(|P(i, j)| * rho + 1e-9)) pairs, rho = rho_1 if
//            L(t) = L0 / 2^B(t) * gamma >= B_s else rho_2 (Eq. 8), drawn
//            uniformly: pair (u, v) gets the 32-bit word (v mod 4) of
//            Philox4x32-10(counter (u, floor(v / 4), i, j), key (seed_lo,
//            seed_hi)) (Salmon et al., SC 2011) and the k pairs with the
//            smallest (word, u * N_t + v) are selected.
//
// Kernels:
//   init:  per frame pair: window, |P| (closed form), k.
//   hist / pick, passes 0-2: radix select of the k-th smallest word, 11 + 11
//          + 10 bits. hist: workgroups of 256 threads over (row chunk, frame
//          pair) regenerate the words of their rows of P(i, j) (one Philox
//          call serves 4 consecutive v) and count, in an LDS histogram, the
//          digit of every word agreeing with the resolved prefix; the
//          non-zero bins are added to the frame pair's global histogram.
//          pick: one workgroup per frame pair scans the histogram, fixes the
//          digit holding the rank and clears the histogram.
//   passes 3-5, only for frame pairs whose k-th word is tied with a word
//          that is not kept: the same on positions u * N_t + v among the pairs
//          with that word. The result is a cut (word T, position p): a pair is
//          selected iff word < T, or word = T and position <= p.
//   mark:  one wavefront per candidate block pair: per lane one query row and
//          16 keys; tiles inside one frame pair with t <= 1 and inside the
//          window are fully selected without any word; the selected bits are
//          counted per key column by ballots and the (theta_c, theta_m) rule
//          is applied with integer thresholds. One flag per candidate entry.
//   compact: flags -> kept lists of every (b, h) (flag_compact_kernel).
#include "dr_internal.h"

namespace dr {
namespace {

constexpr int kChunks = 16;       // row chunks per frame pair in the histogram passes
constexpr int kThreads = 256;

// Philox4x32-10: 10 rounds; round r >= 1 uses the key advanced r times by
// (0x9E3779B9, 0xBB67AE85). Each round maps (c0, c1, c2, c3) to
// (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)) with
// M0 = 0xD2511F53, M1 = 0xCD9E8D57.
__device__ __forceinline__ void philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0, uint32_t k1,
                                       uint32_t out[4]) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c0 = n0;
    c1 = (uint32_t)p1;
    c2 = n2;
    c3 = (uint32_t)p0;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

// digit layout of the six passes: shift and width of the digit being resolved
__host__ __device__ constexpr int pass_shift(int pass) { return pass % 3 == 0 ? 21 : (pass % 3 == 1 ? 10 : 0); }
__host__ __device__ constexpr int pass_bits(int pass) { return pass % 3 == 2 ? 10 : 11; }

__global__ __launch_bounds__(kThreads) void init_kernel(StaticParams p) {
  const int fp = blockIdx.x;
  uint32_t* h = p.hist + (size_t)fp * kStaticBins;
  for (int i = threadIdx.x; i < kStaticBins; i += kThreads) h[i] = 0;
  if (threadIdx.x != 0) return;
  const int i = fp / p.Nf, j = fp - i * p.Nf;
  const int t = i > j ? i - j : j - i;
  int w, sf;
  table_entry(t, p.Nt, p.Bs, p.L0, p.gamma, p.lambda, &w, &sf);
  StaticState st{};
  st.active = (t > 1 && t % sf == 0) ? 1u : 0u;
  const long long wc = w < p.Nt ? w : p.Nt;
  st.w = (uint32_t)wc;
  // |P| = sum over u of the v in [max(0, u - w), min(N_t - 1, u + w)]
  const long long Nt = p.Nt;
  const long long n = wc >= Nt - 1 ? Nt * Nt : Nt * (2 * wc + 1) - wc * (wc + 1);
  st.n = (uint32_t)n;
  if (st.active) {
#pragma clang fp contract(off)
    const int B = 32 - __builtin_clz((unsigned)t);
    const double decay = (double)p.L0 / (double)(1LL << B) * p.gamma;   // Eq. 2, unclamped
    const double rho = decay >= (double)p.Bs ? p.rho_near : p.rho_far;  // Eq. 8
    const double kd = floor((double)n * rho + kCountGuard);
    const long long k = kd < 1.0 ? 1 : (long long)kd;
    st.k = (uint32_t)(k < n ? k : n);
  }
  st.rank = st.k;
  st.group = st.n;
  st.pcut = 0xffffffffu;
  p.state[fp] = st;
}

// Histogram of one pass over the pairs of P(i, j) in this workgroup's rows.
template <int PASS>
__global__ __launch_bounds__(kThreads) void hist_kernel(StaticParams p) {
  constexpr int SHIFT = pass_shift(PASS), BITS = pass_bits(PASS);
  constexpr bool POS = PASS >= 3;
  const int fp = blockIdx.y;
  const StaticState st = p.state[fp];
  if (!st.active || (POS && !st.pos_mode)) return;
  __shared__ uint32_t h[kStaticBins];
  const int tid = threadIdx.x;
  for (int x = tid; x < kStaticBins; x += kThreads) h[x] = 0;
  __syncthreads();
  const int i = fp / p.Nf, j = fp - i * p.Nf;
  const int Nt = p.Nt, w = (int)st.w;
  const int r0 = (int)((long long)blockIdx.x * Nt / kChunks), r1 = (int)((long long)(blockIdx.x + 1) * Nt / kChunks);
  // threads per row: a power of two covering the row's 4-key groups
  const int gw = (min(Nt - 1, 2 * w) >> 2) + 2;
  int tr = 1;
  while (tr < gw && tr < kThreads) tr <<= 1;
  const int rows_per_it = kThreads / tr;
  const uint32_t above = SHIFT + BITS >= 32 ? 0u : ~0u << (SHIFT + BITS);
  for (int u = r0 + tid / tr; u < r1; u += rows_per_it) {
    const int lo = max(0, u - w), hi = min(Nt - 1, u + w);
    for (int g = (lo >> 2) + (tid & (tr - 1)); g <= (hi >> 2); g += tr) {
      uint32_t x[4];
      philox((uint32_t)u, (uint32_t)g, (uint32_t)i, (uint32_t)j, p.seed_lo, p.seed_hi, x);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = 4 * g + e;
        if (v < lo || v > hi) continue;
        uint32_t key;
        if (!POS) {
          if ((x[e] & above) != (st.xpre & above)) continue;
          key = x[e];
        } else {
          const uint32_t pos = (uint32_t)u * (uint32_t)Nt + (uint32_t)v;
          if (x[e] != st.xpre || (pos & above) != (st.ppre & above)) continue;
          key = pos;
        }
        atomicAdd(&h[(key >> SHIFT) & ((1u << BITS) - 1u)], 1u);
      }
    }
  }
  __syncthreads();
  uint32_t* gh = p.hist + (size_t)fp * kStaticBins;
  for (int x = tid; x < kStaticBins; x += kThreads)
    if (h[x]) atomicAdd(&gh[x], h[x]);
}

// Fix the digit holding the rank; clear the histogram for the next pass.
template <int PASS>
__global__ __launch_bounds__(kThreads) void pick_kernel(StaticParams p) {
  constexpr int SHIFT = pass_shift(PASS), BITS = pass_bits(PASS);
  constexpr bool POS = PASS >= 3;
  constexpr int PER = kStaticBins / kThreads;   // 8 bins per thread
  const int fp = blockIdx.x, tid = threadIdx.x;
  __shared__ StaticState st;
  __shared__ uint32_t part[kThreads];
  if (tid == 0) st = p.state[fp];
  __syncthreads();
  if (!st.active || (POS && !st.pos_mode)) return;
  uint32_t* gh = p.hist + (size_t)fp * kStaticBins;
  uint32_t b[PER];
  uint32_t sum = 0;
#pragma unroll
  for (int x = 0; x < PER; ++x) {
    b[x] = gh[tid * PER + x];
    sum += b[x];
  }
  part[tid] = sum;
  __syncthreads();
  // inclusive scan of the per-thread sums (Hillis-Steele in LDS)
  for (int off = 1; off < kThreads; off <<= 1) {
    const uint32_t add = tid >= off ? part[tid - off] : 0u;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  const uint32_t incl = part[tid], excl = incl - sum;
  if (excl < st.rank && st.rank <= incl) {
    // first bin of this thread whose inclusive count reaches the rank
    uint32_t run = excl;
    int d = -1;
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      if (d < 0 && run + b[x] >= st.rank) d = x;
      if (d < 0) run += b[x];
    }
    const uint32_t digit = (uint32_t)(tid * PER + d);
    StaticState s = st;
    s.rank -= run;
#pragma unroll
    for (int x = 0; x < PER; ++x)
      if (x == d) s.group = b[x];
    if (!POS) s.xpre |= digit << SHIFT;
    else s.ppre |= digit << SHIFT;
    if (PASS == 2) {
      // the k-th word is T = xpre; if every pair with word T is kept, no
      // position cut is needed
      if (s.rank == s.group) {
        s.pcut = 0xffffffffu;
        s.pos_mode = 0;
      } else {
        s.pos_mode = 1;
      }
    }
    if (PASS == 5) s.pcut = s.ppre;
    p.state[fp] = s;
  }
  (void)BITS;
#pragma unroll
  for (int x = 0; x < PER; ++x) gh[tid * PER + x] = 0;
}

// One wavefront per candidate block pair; 4 wavefronts per workgroup, one
// workgroup per query block.
template <int BS>
__global__ __launch_bounds__(kThreads) void mark_kernel(StaticParams p) {
  constexpr int FRMAX = BS / 32 + 1;   // query frames a block can touch (N_t >= 32)
  const int a = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int s_w[kMaxTokenFrames], s_sf[kMaxTokenFrames];
  __shared__ uint32_t s_T[FRMAX * kMaxTokenFrames], s_P[FRMAX * kMaxTokenFrames];
  __shared__ int min_c[BS + 1], min_a[BS + 1];
  const int Nf = p.Nf, Nt = p.Nt, S = p.S;
  const int f_lo = (a * BS) / Nt;
  for (int t = tid; t < Nf; t += kThreads) {
    int w, sf;
    table_entry(t, Nt, BS, p.L0, p.gamma, p.lambda, &w, &sf);
    s_w[t] = w < Nt ? w : Nt;
    s_sf[t] = sf;
  }
  for (int x = tid; x < FRMAX * Nf; x += kThreads) {
    const int fq = f_lo + x / Nf, fk = x % Nf;
    uint32_t T = 0, P = 0;
    if (fq < Nf) {
      const StaticState st = p.state[fq * Nf + fk];
      T = st.xpre;
      P = st.pcut;
    }
    s_T[x] = T;
    s_P[x] = P;
  }
  for (int n = 1 + tid; n <= BS; n += kThreads) {
    min_c[n] = min_count(n, p.theta_c);
    min_a[n] = min_count(n, p.theta_m);
  }
  __syncthreads();
  const int nq = min(BS, S - a * BS);
  const int e0 = p.row_ptr[a], e1 = p.row_ptr[a + 1];
  const int r = lane & 31, kh = 16 * (lane >> 5);
  for (int e = e0 + wave; e < e1; e += kThreads / 64) {
    const int b = p.cols[e];
    const int nk = min(BS, S - b * BS);
    int cnt = 0, cnt_hi = 0;   // lane c: selected count of key columns c and 64 + c of the block
#pragma unroll
    for (int qt = 0; qt < BS / 32; ++qt) {
#pragma unroll
      for (int kt = 0; kt < BS / 32; ++kt) {
        const int q0 = a * BS + 32 * qt, k0 = b * BS + 32 * kt;
        if (q0 >= S || k0 >= S) continue;
        // whole-tile classes (scalar): one frame pair, t <= 1, inside the window
        bool all = false, none = false;
        if (q0 + 31 < S && k0 + 31 < S) {
          const int fq = q0 / Nt, fk = k0 / Nt;
          if ((q0 + 31) / Nt == fq && (k0 + 31) / Nt == fk) {
            const int t = fq > fk ? fq - fk : fk - fq;
            const int uq = q0 - fq * Nt, uk = k0 - fk * Nt, w = s_w[t];
            const int dmax = max(uq + 31 - uk, uk + 31 - uq);
            const int dmin = max(0, max(uk - (uq + 31), uq - (uk + 31)));
            if (t % s_sf[t] != 0 || dmin > w) none = true;
            else if (t <= 1 && dmax <= w) all = true;
          }
        }
        if (none) continue;
        uint32_t bits = 0;   // this lane's row against keys kh .. kh + 15
        if (all) {
          bits = 0xffffu;
        } else {
          const int q = q0 + r;
          if (q < S) {
            const int fq = q / Nt, u = q - fq * Nt;
            int k = k0 + kh;
            int fk = k / Nt, v = k - fk * Nt;
            int cg = -1, cf = -1;
            uint32_t x[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int c = 0; c < 16; ++c, ++k, ++v) {
              if (v == Nt) {
                v = 0;
                ++fk;
              }
              if (k >= S) break;
              const int t = fq > fk ? fq - fk : fk - fq;
              const int du = u > v ? u - v : v - u;
              if (t % s_sf[t] != 0 || du > s_w[t]) continue;
              bool sel = t <= 1;
              if (!sel) {
                if ((v >> 2) != cg || fk != cf) {
                  cg = v >> 2;
                  cf = fk;
                  philox((uint32_t)u, (uint32_t)cg, (uint32_t)fq, (uint32_t)fk, p.seed_lo, p.seed_hi, x);
                }
                const uint32_t word = x[v & 3];
                const int slot = (fq - f_lo) * Nf + fk;
                const uint32_t T = s_T[slot];
                sel = word < T || (word == T && (uint32_t)u * (uint32_t)Nt + (uint32_t)v <= s_P[slot]);
              }
              if (sel) bits |= 1u << c;
            }
          }
        }
        // column counts: key c of half h is column 32 kt + kh + c
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const unsigned long long m = __ballot((bits >> c) & 1u);
          const int lo = __popcll(m & 0xffffffffull), hi = __popcll(m >> 32);
          const int col = 32 * kt + c;   // (+16 for the upper half-wave's keys)
          if (col < 64) {
            if (lane == col) cnt += lo;
            if (lane == col + 16) cnt += hi;
          } else {
            if (lane == col - 64) cnt_hi += lo;
            if (lane == col - 48) cnt_hi += hi;
          }
        }
      }
    }
    const int n_act = __popcll(__ballot(lane < nk && cnt >= min_c[nq])) +
                      (BS > 64 ? __popcll(__ballot(64 + lane < nk && cnt_hi >= min_c[nq])) : 0);
    if (lane == 0) p.flags[e] = n_act >= min_a[nk] ? 1 : 0;
  }
}

template <int BS>
hipError_t launch_all(const StaticParams& p, hipStream_t stream) {
  const int nfp = p.Nf * p.Nf;
  hipLaunchKernelGGL(init_kernel, dim3((unsigned)nfp), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 hgrid(kChunks, (unsigned)nfp);
#define DR_STATIC_PASS(P)                                                                         \
  hipLaunchKernelGGL(hist_kernel<P>, hgrid, dim3(kThreads), 0, stream, p);                        \
  if ((e = hipGetLastError()) != hipSuccess) return e;                                            \
  hipLaunchKernelGGL(pick_kernel<P>, dim3((unsigned)nfp), dim3(kThreads), 0, stream, p);         \
  if ((e = hipGetLastError()) != hipSuccess) return e;
  DR_STATIC_PASS(0)
  DR_STATIC_PASS(1)
  DR_STATIC_PASS(2)
  DR_STATIC_PASS(3)
  DR_STATIC_PASS(4)
  DR_STATIC_PASS(5)
#undef DR_STATIC_PASS
  hipLaunchKernelGGL(mark_kernel<BS>, dim3((unsigned)p.Sb), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_static_select(const StaticParams& p, hipStream_t stream) {
  if (p.Bs == 32) return launch_all<32>(p, stream);
  if (p.Bs == 64) return launch_all<64>(p, stream);
  if (p.Bs == 128) return launch_all<128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace dr
