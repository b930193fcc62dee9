// Choice of the query-block grouping of the sparse attention, per (b, h).
//
// A workgroup of the sparse attention streams the union of its query blocks'
// kept key blocks through LDS ([DR] §3.3: every kept block pair is one tile of
// the flash-style attention), so the bytes it reads from past L2 grow with the
// size of that union. For each grouping mode (consecutive blocks, or blocks at
// the same place in neighbouring frames) the union sizes of every
// kGroupSample-th group of a (b, h) are summed and scaled to the mode's group
// count; the mode with the smallest estimate (ties: the lower mode) is
// written. Integer work (the comparison cross-multiplied), deterministic. The
// grouping sets the attention's memory traffic; its outputs agree under every
// grouping up to the order of accumulation.
//
// The same kernels also run on a library-held scratch array instead of a
// caller workspace (group_scratch), for callers that cannot allocate.
#include "dr_internal.h"

#include <mutex>

namespace dr {
namespace {

constexpr int kThreads = 256;
constexpr int kGroupSample = 4;   // every 4th group of a mode is measured

__global__ __launch_bounds__(kThreads) void zero_kernel(uint32_t* x, int n) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) x[i] = 0;
}

// One wavefront per (group, mode, b, h) (4 per workgroup, no workgroup
// barrier): the union of the group's kept lists as a bitmap over key blocks in
// the wave's own LDS words, its population added to the mode's total. LDS
// operations of a wavefront complete in issue order.
__global__ __launch_bounds__(kThreads) void union_kernel(GroupCostParams p) {
  extern __shared__ unsigned int s_bits[];
  const int nword = (p.grp.Sb + 31) >> 5;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long item = (long long)blockIdx.x * (kThreads / 64) + wave;
  const long long per_bh = (long long)p.gmax * kGroupModes;
  if (item >= per_bh * p.BH) return;
  const int bh = (int)(item / per_bh);
  const int r = (int)(item - (long long)bh * per_bh);
  const int mode = r % kGroupModes, g = r / kGroupModes;
  if (g >= group_count(p.grp, mode) || g % kGroupSample != 0) return;
  unsigned int* bits = s_bits + wave * nword;
  for (int i = lane; i < nword; i += 64) bits[i] = 0;
  // slot s of the group: lane s holds its list's start and length
  int start = 0, cnt = 0;
  if (lane < p.grp.QB) {
    const int qb = group_block(p.grp, mode, g, lane);
    if (qb >= 0) {
      start = p.row_ptr[qb];
      cnt = min(p.kept_cnt[(long long)bh * p.grp.Sb + qb], p.row_ptr[qb + 1] - start);
    }
  }
  const int32_t* base = p.kept_col + (long long)bh * p.nnz;
  for (int s = 0; s < p.grp.QB; ++s) {
    const int st = __shfl(start, s), n = __shfl(cnt, s);
    for (int i = lane; i < n; i += 64) {
      const int c = base[st + i];
      if (c >= 0 && c < p.grp.Sb) atomicOr(&bits[c >> 5], 1u << (c & 31));
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  unsigned int n = 0;
  for (int i = lane; i < nword; i += 64) n += __popc(bits[i]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) n += __shfl_xor(n, off);
  if (lane == 0) atomicAdd(&p.totals[bh * kGroupModes + mode], n);
}

__global__ __launch_bounds__(kThreads) void choose_kernel(GroupCostParams p) {
  const int bh = blockIdx.x * kThreads + threadIdx.x;
  if (bh >= p.BH) return;
  // estimate of mode m: t_m * count_m / sampled_m; compared as
  // t_a * count_a * sampled_b < t_b * count_b * sampled_a
  auto sampled = [&](int m) -> unsigned long long {
    return (unsigned long long)((group_count(p.grp, m) + kGroupSample - 1) / kGroupSample);
  };
  int best = 0;
  unsigned long long bt = p.totals[bh * kGroupModes], bc = (unsigned long long)group_count(p.grp, 0),
                     bs = sampled(0);
  for (int m = 1; m < kGroupModes; ++m) {
    if (group_count(p.grp, m) == 0) continue;
    const unsigned long long t = p.totals[bh * kGroupModes + m], c = (unsigned long long)group_count(p.grp, m),
                             s = sampled(m);
    if (t * c * bs < bt * bc * s) {
      best = m;
      bt = t;
      bc = c;
      bs = s;
    }
  }
  p.group_mode[bh] = best;
}

// Union totals of every (b, h) and mode for the entry point that allocates
// nothing: one array per GPU for the life of the process. Calls on one GPU
// share it, so calls that overlap on one GPU race.
__device__ __align__(256) uint32_t g_group_scratch[kGroupScratchBH * kGroupModes];

}  // namespace

hipError_t group_scratch(uint32_t** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static uint32_t* ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    // the array's device address on the current device (the host-side name is
    // only a stand-in, never a device address)
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(g_group_scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = static_cast<uint32_t*>(a);
  }
  *out = ptr[dev];
  return hipSuccess;
}

hipError_t launch_group_choice(const GroupCostParams& p, hipStream_t stream) {
  const int n = p.BH * kGroupModes;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream,
                     p.totals, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)(kThreads / 64) * ((p.grp.Sb + 31) / 32) * 4;
  const long long items = (long long)p.gmax * kGroupModes * p.BH;
  hipLaunchKernelGGL(union_kernel, dim3((unsigned)((items + kThreads / 64 - 1) / (kThreads / 64))), dim3(kThreads),
                     lds, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(choose_kernel, dim3((unsigned)((p.BH + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream,
                     p);
  return hipGetLastError();
}

}  // namespace dr
