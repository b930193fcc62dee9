// Radial block-candidate set on gfx950 ([DR] §3.1, Eqs. 1-7 and
// "Density control within blocks"; [DR] = "DynamicRad: Content-Adaptive Sparse
// Attention for Long Video Diffusion", arXiv 2604.20470).
//
// Integer work, content-free. Three launches, no scratch memory:
//   count: one workgroup per query block a evaluates every key block b and
//          writes the row's candidate count into row_ptr[a + 1];
//   scan:  one workgroup turns the counts into the CSR row pointer in place;
//   fill:  one workgroup per query block re-evaluates its row and writes the
//          ascending key-block indices with an ordered workgroup compaction.
// Each workgroup first builds the per-distance table (w(t), sf(t)) in LDS
// from the same double-precision expression the host uses.
#include "dr_internal.h"

namespace dr {
namespace {

constexpr int kCandThreads = 256;

__device__ void build_table(const CandParams& p, int* s_w, int* s_sf) {
  for (int t = threadIdx.x; t < p.Nf; t += blockDim.x) {
    int w, sf;
    table_entry(t, p.Nt, p.Bs, p.L0, p.gamma, p.lambda, &w, &sf);
    // |u - v| <= N_t - 1 always, so any window >= N_t admits every pair.
    s_w[t] = w < p.Nt ? w : p.Nt;
    s_sf[t] = sf;
  }
}

// Is (query block a, key block b) a candidate? Token pair (q, k) is a candidate
// iff t = |f_q - f_k| has t mod sf(t) == 0 (Eq. 6) and |u_q - u_k| <= w(t) (Eq. 7).
// For each key token k of b, the query tokens of a paired with it are counted
// per frame segment of a as an interval intersection. Column k is active iff
// count / n_q > theta_c; the block is a candidate iff active / n_k > theta_m.
// active only grows, so the first time the block test passes decides it.
__device__ bool is_candidate(int a, int b, const CandParams& p, const int* s_w, const int* s_sf, const int* s_thr) {
  const int q0 = a * p.Bs, q1 = min(q0 + p.Bs, p.S);
  const int k0 = b * p.Bs, k1 = min(k0 + p.Bs, p.S);
  // Some query frame segment and some key frame segment retained (Eq. 6) and
  // within w(t) of each other (Eq. 7; the interval distance
  // max(0, v_lo - u_hi, u_lo - v_hi) decides it) is necessary for any token
  // pair, and with both thresholds at 0 it is also sufficient.
  bool near = false;
  for (int s = q0; s < q1 && !near;) {
    const int fq = s / p.Nt;
    const int s_end = min(q1, (fq + 1) * p.Nt);
    const int ulo = s - fq * p.Nt, uhi = s_end - 1 - fq * p.Nt;
    for (int k = k0; k < k1;) {
      const int fk = k / p.Nt;
      const int k_end = min(k1, (fk + 1) * p.Nt);
      const int vlo = k - fk * p.Nt, vhi = k_end - 1 - fk * p.Nt;
      const int t = fq > fk ? fq - fk : fk - fq;
      if (t % s_sf[t] == 0 && max(0, max(vlo - uhi, ulo - vhi)) <= s_w[t]) {
        near = true;
        break;
      }
      k = k_end;
    }
    s = s_end;
  }
  if (!near || (p.theta_c == 0.0 && p.theta_m == 0.0)) return near;
  // the shares count / n_q > theta_c and active / n_k > theta_m as integer
  // thresholds (min_count: exact, a correctly rounded quotient being monotone)
  const int thr_c = s_thr[0];
  const int thr_m = k1 - k0 == p.Bs ? s_thr[1] : s_thr[2];
  int active = 0;
  if (q0 / p.Nt == (q1 - 1) / p.Nt) {
    // One query frame segment [u_lo, u_hi]: within a key frame segment the
    // count of column u_k is |[u_lo, u_hi] n [u_k - w, u_k + w]|, which is at
    // least c iff c <= n_q, c <= 2w + 1, u_k >= u_lo + c - 1 - w and
    // u_k <= u_hi - c + 1 + w, so the active columns form one interval.
    const int fq = q0 / p.Nt;
    const int ulo = q0 - fq * p.Nt, uhi = q1 - 1 - fq * p.Nt;
    const int nq = q1 - q0;
    for (int k = k0; k < k1;) {
      const int fk2 = k / p.Nt;
      const int k_end = min(k1, (fk2 + 1) * p.Nt);
      const int vlo = k - fk2 * p.Nt, vhi = k_end - 1 - fk2 * p.Nt;
      const int t = fq > fk2 ? fq - fk2 : fk2 - fq;
      const int w = s_w[t];
      if (t % s_sf[t] == 0 && thr_c <= nq && thr_c <= 2 * w + 1) {
        const int lo = max(vlo, ulo + thr_c - 1 - w), hi = min(vhi, uhi - thr_c + 1 + w);
        if (hi >= lo) active += hi - lo + 1;
      }
      k = k_end;
    }
    return active >= thr_m;
  }
  int fk = k0 / p.Nt, uk = k0 - fk * p.Nt;
  for (int k = k0; k < k1; ++k, ++uk) {
    if (uk == p.Nt) {
      ++fk;
      uk = 0;
    }
    int cnt = 0;
    for (int s = q0; s < q1;) {
      const int fq = s / p.Nt;
      const int seg_end = min(q1, (fq + 1) * p.Nt);
      const int t = fq > fk ? fq - fk : fk - fq;
      if (t % s_sf[t] == 0) {
        const int w = s_w[t];
        const int lo = max(s - fq * p.Nt, uk - w);
        const int hi = min(seg_end - 1 - fq * p.Nt, uk + w);
        if (hi >= lo) cnt += hi - lo + 1;
      }
      s = seg_end;
    }
    if (cnt >= thr_c && ++active >= thr_m) return true;
    if (active + (k1 - 1 - k) < thr_m) return false;   // the remaining columns cannot reach it
  }
  return false;
}

// Integer thresholds of the density control for this query block: [0] the
// active-column count for its n_q queries, [1] the candidate test for a full
// key block, [2] for the last (possibly ragged) key block.
__device__ void build_thresholds(const CandParams& p, int a, int* s_thr) {
  const int nq = min(p.Bs, p.S - a * p.Bs);
  const int nk_last = p.S - (p.Sb - 1) * p.Bs;
  if (threadIdx.x == 0) s_thr[0] = min_count(nq, p.theta_c);
  if (threadIdx.x == 1) s_thr[1] = min_count(p.Bs, p.theta_m);
  if (threadIdx.x == 2) s_thr[2] = min_count(nk_last, p.theta_m);
}

__global__ __launch_bounds__(kCandThreads) void cand_count_kernel(CandParams p, int32_t* row_ptr) {
  extern __shared__ int s_tab[];
  int* s_w = s_tab;
  int* s_sf = s_tab + p.Nf;
  __shared__ int s_part[kCandThreads / 64];
  __shared__ int s_thr[3];
  const int a = blockIdx.x;
  build_table(p, s_w, s_sf);
  build_thresholds(p, a, s_thr);
  __syncthreads();
  int cnt = 0;
  for (int b = threadIdx.x; b < p.Sb; b += kCandThreads) cnt += is_candidate(a, b, p, s_w, s_sf, s_thr) ? 1 : 0;
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    int tot = 0;
    for (int w = 0; w < kCandThreads / 64; ++w) tot += s_part[w];
    row_ptr[a + 1] = tot;
    if (a == 0) row_ptr[0] = 0;
  }
}

// In-place inclusive scan of row_ptr[1 .. n] by one workgroup of 1024 threads.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void scan_kernel(int32_t* row_ptr, int n) {
  __shared__ int s_sum[kScanThreads];
  int32_t* x = row_ptr + 1;
  const int per = (n + kScanThreads - 1) / kScanThreads;
  const int lo = min(n, (int)threadIdx.x * per), hi = min(n, lo + per);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += x[i];
  s_sum[threadIdx.x] = local;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int v = threadIdx.x >= (unsigned)off ? s_sum[threadIdx.x - off] : 0;
    __syncthreads();
    s_sum[threadIdx.x] += v;
    __syncthreads();
  }
  int run = s_sum[threadIdx.x] - local;   // exclusive prefix of this thread's chunk
  for (int i = lo; i < hi; ++i) {
    run += x[i];
    x[i] = run;
  }
}

__global__ __launch_bounds__(kCandThreads) void cand_fill_kernel(CandParams p, const int32_t* row_ptr,
                                                                 int32_t* cols, long long cap) {
  extern __shared__ int s_tab[];
  int* s_w = s_tab;
  int* s_sf = s_tab + p.Nf;
  __shared__ int s_wave[kCandThreads / 64];
  __shared__ int s_thr[3];
  const int a = blockIdx.x;
  build_table(p, s_w, s_sf);
  build_thresholds(p, a, s_thr);
  __syncthreads();
  const int wave = threadIdx.x >> 6;
  long long base = row_ptr[a];
  for (int b0 = 0; b0 < p.Sb; b0 += kCandThreads) {
    const int b = b0 + (int)threadIdx.x;
    const bool flag = b < p.Sb && is_candidate(a, b, p, s_w, s_sf, s_thr);
    const unsigned long long m = __ballot(flag);
    const int before = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0));
    if ((threadIdx.x & 63) == 0) s_wave[wave] = __popcll(m);
    __syncthreads();
    int off = 0, tot = 0;
    for (int w = 0; w < kCandThreads / 64; ++w) {
      const int c = s_wave[w];
      off += w < wave ? c : 0;
      tot += c;
    }
    const long long pos = base + off + before;
    if (flag && pos < cap) cols[pos] = b;
    base += tot;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_candidates(const CandParams& p, int32_t* row_ptr, int32_t* cols, long long cap,
                             hipStream_t stream) {
  const size_t tab_bytes = 2 * (size_t)p.Nf * sizeof(int);
  hipLaunchKernelGGL(cand_count_kernel, dim3(p.Sb), dim3(kCandThreads), tab_bytes, stream, p, row_ptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, row_ptr, p.Sb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cand_fill_kernel, dim3(p.Sb), dim3(kCandThreads), tab_bytes, stream, p,
                     (const int32_t*)row_ptr, cols, cap);
  return hipGetLastError();
}

}  // namespace dr
