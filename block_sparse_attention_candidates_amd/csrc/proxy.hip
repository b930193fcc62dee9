// Proxy-task error sums on gfx950 ([DR] App. C.4 "Optimization Objective",
// Eq. 22, evaluated through a random probe). [DR] = "DynamicRad:
// Content-Adaptive Sparse Attention for Long Video Diffusion", arXiv 2604.20470.
//
// Given the dense output O = A Z and the kept-block output O' = A' Z of one
// probe Z, the normalised squared error of Eq. 22 is estimated by
// sum (O' - O)^2 / sum O^2; the sparsity term needs the number of kept block
// pairs, the sum of the kept counts. Both are plain reductions bound by HBM:
// every bf16 element is read once with 16-byte loads. Each thread sums a fixed
// grid-strided set of elements in float64, workgroups reduce in a fixed tree
// order into one partial each, and a single workgroup adds the partials in
// order, so the result is bit-reproducible. With the loss requested, the same
// workgroup also forms Eq. 22 from the three sums: the normalised error, the
// sparsity 1 - (kept block pairs) / (all block pairs) and the penalised loss.
#include "dr_internal.h"

namespace dr {
namespace {

constexpr int kThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double bf16_lo(unsigned int w) { return (double)__uint_as_float(w << 16); }
__device__ __forceinline__ double bf16_hi(unsigned int w) { return (double)__uint_as_float(w & 0xffff0000u); }

// Sum of three values over the workgroup, in a fixed order: wavefront trees,
// then wave 0 adds the four wave results in order.
__device__ __forceinline__ void block_sum3(double& a, double& b, double& c) {
  __shared__ double part[3][kThreads / 64];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    a += __shfl_xor(a, off);
    b += __shfl_xor(b, off);
    c += __shfl_xor(c, off);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    part[0][wave] = a;
    part[1][wave] = b;
    part[2][wave] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a = b = c = 0.0;
    for (int w = 0; w < kThreads / 64; ++w) {
      a += part[0][w];
      b += part[1][w];
      c += part[2][w];
    }
  }
}

__global__ __launch_bounds__(kThreads) void partial_kernel(ProxyParams p) {
  const long long tid = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long stride = (long long)gridDim.x * kThreads;
  double d2 = 0.0, r2 = 0.0, cnt = 0.0;
  // 8 elements (16 bytes) per step; both operands are 16-byte aligned
  const long long n8 = p.n / 8;
  const u32x4* ref8 = reinterpret_cast<const u32x4*>(p.ref);
  const u32x4* test8 = reinterpret_cast<const u32x4*>(p.test);
  for (long long i = tid; i < n8; i += stride) {
    const u32x4 r = ref8[i], t = test8[i];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const double rl = bf16_lo(r[w]), rh = bf16_hi(r[w]);
      const double dl = bf16_lo(t[w]) - rl, dh = bf16_hi(t[w]) - rh;
      d2 += dl * dl + dh * dh;
      r2 += rl * rl + rh * rh;
    }
  }
  for (long long i = n8 * 8 + tid; i < p.n; i += stride) {
    const double r = (double)__uint_as_float((unsigned int)p.ref[i] << 16);
    const double d = (double)__uint_as_float((unsigned int)p.test[i] << 16) - r;
    d2 += d * d;
    r2 += r * r;
  }
  for (long long i = tid; i < p.n_cnt; i += stride) cnt += (double)p.kept_cnt[i];
  block_sum3(d2, r2, cnt);
  if (threadIdx.x == 0) {
    p.partial[3 * blockIdx.x + 0] = d2;
    p.partial[3 * blockIdx.x + 1] = r2;
    p.partial[3 * blockIdx.x + 2] = cnt;
  }
}

__global__ __launch_bounds__(kThreads) void final_kernel(ProxyParams p) {
  double d2 = 0.0, r2 = 0.0, cnt = 0.0;
  for (int i = threadIdx.x; i < kProxyPartials; i += kThreads) {
    d2 += p.partial[3 * i + 0];
    r2 += p.partial[3 * i + 1];
    cnt += p.partial[3 * i + 2];
  }
  block_sum3(d2, r2, cnt);
  if (threadIdx.x == 0) {
    p.out[0] = d2;
    p.out[1] = r2;
    p.out[2] = cnt;
    if (p.with_loss) {
      // Eq. 22: normalised squared error plus the sparsity shortfall penalty
      const double nmse = d2 / r2;
      const double sparsity = 1.0 - cnt / (double)p.total_blocks;
      const double shortfall = p.target - sparsity;
      p.out[3] = nmse;
      p.out[4] = sparsity;
      p.out[5] = nmse + p.alpha * (shortfall > 0.0 ? shortfall : 0.0);
    }
  }
}

}  // namespace

hipError_t launch_proxy_error(const ProxyParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(partial_kernel, dim3(kProxyPartials), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(final_kernel, dim3(1), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dr
