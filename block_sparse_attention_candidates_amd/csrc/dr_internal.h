// Internal declarations shared by the C ABI (api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dr {

constexpr int kMaxFrames = 4096;     // N_f limit (per-distance table in LDS)
constexpr int kMaxBlocks = 16384;    // S_b limit (LDS bitmaps / selection rows)
constexpr int kWindowCap = 1 << 30;  // saturation of w(t) and sf(t)
constexpr double kSplitEps = 1e-6;   // epsilon of [DR] Eq. 5
constexpr double kCountGuard = 1e-9; // ceil(r * n - guard) in the static count

// Next power of two >= n ([DR] §3.1 Eq. 1, L0).
__host__ __device__ inline int base_span(int n) {
  int L0 = 1;
  while (L0 < n) L0 <<= 1;
  return L0;
}

// One entry of the per-distance table, [DR] §3.1 Eqs. 1-5.
// t = 0: dense (w = N_t, sf = 1). t >= 1: B = floor(log2 t) + 1 (bit length),
// span = L0 / 2^B, L = span * gamma (Eq. 2), w = N_t if t == 1 else
// max(B_s, floor(L + 1/2)) (Eq. 3), sf = max(1, floor(B_s / (span * lambda + eps)))
// (Eqs. 4-5). IEEE double, operations in this order, never contracted into FMAs,
// so host and device produce identical tables.
__host__ __device__ inline void table_entry(int t, int Nt, int Bs, int L0, double gamma,
                                            double lambda, int* w, int* sf) {
#pragma clang fp contract(off)
  if (t == 0) {
    *w = Nt;
    *sf = 1;
    return;
  }
  const int B = 32 - __builtin_clz((unsigned)t);
  const double span = (double)L0 / (double)(1LL << B);
  const double decay = span * gamma;
  int ww;
  if (t <= 1) {
    ww = Nt;
  } else {
    const double r = floor(decay + 0.5);
    ww = r >= (double)kWindowCap ? kWindowCap : (int)r;
    if (ww < Bs) ww = Bs;
  }
  const double split = span * lambda;
  const double qd = floor((double)Bs / (split + kSplitEps));
  const int s = qd >= (double)kWindowCap ? kWindowCap : (int)qd;
  *w = ww;
  *sf = s < 1 ? 1 : s;
}

// Density-control decision by integer thresholds ([DR] §3.1 "Density control
// within blocks"): the smallest count c in [0, n] with (double) c / n > theta
// (n + 1 if none). A correctly rounded quotient is monotone in c, so
// c >= min_count(n, theta) holds exactly when the float64 comparison does.
__host__ __device__ inline int min_count(int n, double theta) {
  int c = 0;
  while (c <= n && !((double)c / (double)n > theta)) ++c;
  return c;
}

// Workgroups go to the 8 XCDs round-robin in dispatch order, and each XCD has
// its own L2. This maps dispatch index L of n to a work index such that every
// XCD receives one contiguous range of the work.
constexpr int kXcds = 8;
__device__ inline int xcd_contiguous(int L, int n) {
  const int x = L % kXcds, i = L / kXcds, q = n / kXcds, r = n % kXcds;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// The same dispatch order mapped so that runs of C consecutive work items land
// on one XCD at about the same time, while successive runs go to successive
// XCDs (so every XCD still sweeps the whole range, in step with the others).
// Work items past the last full round of kXcds * C runs keep their index.
__device__ inline int xcd_chunked(int L, int n, int C) {
  const int round = kXcds * C;
  if (L >= n / round * round) return L;
  const int x = L % kXcds, i = L / kXcds;
  return ((i / C) * kXcds + x) * C + i % C;
}

struct CandParams {
  int Nf, Nt, Bs, S, Sb, L0;
  double gamma, lambda, theta_c, theta_m;
};

struct PoolParams {
  const uint16_t* q;
  const uint16_t* k;
  float* qbar;     // [B, Hp, S_b, D]
  float* kbar;
  int B, H, Hp;    // Hp: heads pooled (H, or the fused-head count)
  int S, Sb, Bs, D;
};

// Head-independent description of the candidate tiles of each group of 32
// consecutive query blocks: the 32-block words (key tiles) holding a candidate
// of any of the group's rows, and per tile and row the candidate bitmap and the
// CSR position of the word's first candidate.
struct TileDesc {
  int32_t* count;   // [ngroups] active tiles
  int32_t* word;    // [ngroups][nword] key tile of active tile j
  uint32_t* bits;   // [ngroups][nword][32] row bitmaps of active tile j
  int32_t* pos;     // [ngroups][nword][32] CSR position of its first candidate
  int ngroups, nword;
};

struct ScoreParams {
  const float* qbar;
  const float* kbar;
  const int32_t* row_ptr;
  const int32_t* cols;
  float* scores;   // [B * Hm * nnz]
  TileDesc tiles;
  long long nnz;
  int Sb, Hp, Hm, g;  // g heads summed per score (1: per-head)
  int D;
  float scale;     // 1 / (sqrt(D) * g)
};

struct SelectParams {
  const float* scores;
  const int32_t* row_ptr;
  const int32_t* cols;
  int32_t* kept_col;
  int32_t* kept_cnt;
  long long nnz;
  int Sb, H, Hm;
  int mode;
  double ratio, tau;
  int max_row;     // longest row (bounds the per-wave register and LDS capacity)
  int min_n;       // rows of at most min_n candidates are left to the per-wave kernel
};

// Query-block grouping of the sparse attention: a workgroup owns QB = 256 / B_s
// query blocks, and the blocks of one (b, h) are partitioned into groups of at
// most QB. Mode 0 groups consecutive blocks (QB g .. QB g + QB - 1). Modes 1 and
// 2 lay the blocks out in rows, one per frame (row f holds blocks
// [floor(f N_t / B_s), floor((f + 1) N_t / B_s)), the last row runs to S_b),
// and group g takes F consecutive rows by R adjacent columns (F R = QB): blocks
// at the same place in neighbouring frames, whose kept lists tend to share key
// blocks when the selection follows content. Every mode is a partition of
// [0, S_b); a mode without a shape for this QB has no groups.
constexpr int kGroupModes = 3;

struct QGroup {
  int QB, Nf, Nt, Bs, Sb;
  int cols[kGroupModes];   // column chunks per row chunk (modes 1, 2)
};

__host__ __device__ inline void group_shape(int QB, int mode, int* F, int* R) {
  // QB = 2, 4, 8 -> index 0, 1, 2
  const int i = QB == 2 ? 0 : QB == 4 ? 1 : 2;
  const int f1[3] = {2, 2, 4}, r1[3] = {1, 2, 2}, f2[3] = {0, 4, 2}, r2[3] = {0, 1, 4};
  *F = mode == 1 ? f1[i] : mode == 2 ? f2[i] : 0;
  *R = mode == 1 ? r1[i] : mode == 2 ? r2[i] : 0;
}

__host__ __device__ inline int frame_row_start(const QGroup& q, int f) {
  return (int)(((long long)f * q.Nt) / q.Bs);
}

__host__ __device__ inline int frame_row_end(const QGroup& q, int f) {
  return f == q.Nf - 1 ? q.Sb : frame_row_start(q, f + 1);
}

// Groups of a mode (0 for a mode without a shape).
__host__ __device__ inline int group_count(const QGroup& q, int mode) {
  if (mode == 0) return (q.Sb + q.QB - 1) / q.QB;
  int F, R;
  group_shape(q.QB, mode, &F, &R);
  if (F == 0) return 0;
  return ((q.Nf + F - 1) / F) * q.cols[mode];
}

// Query block in slot s of group g (-1: empty slot).
__host__ __device__ inline int group_block(const QGroup& q, int mode, int g, int s) {
  if (mode == 0) {
    const int a = g * q.QB + s;
    return a < q.Sb ? a : -1;
  }
  int F, R;
  group_shape(q.QB, mode, &F, &R);
  if (F == 0) return -1;
  const int rc = g / q.cols[mode], cc = g - rc * q.cols[mode];
  const int f = rc * F + s / R, c = cc * R + s % R;
  if (f >= q.Nf) return -1;
  const int s0 = frame_row_start(q, f);
  return c < frame_row_end(q, f) - s0 ? s0 + c : -1;
}

// Host: the grouping geometry of a layout.
inline QGroup make_qgroup(int Nf, int Nt, int Bs, int Sb) {
  QGroup q;
  q.QB = 256 / Bs;
  q.Nf = Nf;
  q.Nt = Nt;
  q.Bs = Bs;
  q.Sb = Sb;
  int lmax = 0;
  for (int f = 0; f < Nf; ++f) {
    const int len = frame_row_end(q, f) - frame_row_start(q, f);
    if (len > lmax) lmax = len;
  }
  for (int m = 0; m < kGroupModes; ++m) {
    int F, R;
    group_shape(q.QB, m, &F, &R);
    q.cols[m] = R > 0 ? (lmax + R - 1) / R : 0;
  }
  return q;
}

// Bounded waits of the ring protocols: every wait polls at most spin_limit
// times (kDefaultSpinLimit unless a caller lowered it for a test of this
// report). A wave whose wait gives up ORs its bit into its file's flag word in
// device memory (a vector-memory atomic) and goes on, so every kernel still
// exits; the host reads and clears the words with take_wait_flags_*().
constexpr int kDefaultSpinLimit = 1 << 26;
constexpr unsigned kWaitAttnLoader = 1u;    // attention loader: slot refilled before it was free
constexpr unsigned kWaitAttnCompute = 2u;   // attention compute wave: unit read before it was published
constexpr unsigned kWaitToken = 4u;         // token selector: key block read before it was published
hipError_t take_wait_flags_attn(unsigned* flags, hipStream_t stream);
hipError_t take_wait_flags_token(unsigned* flags, hipStream_t stream);

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  const int32_t* row_ptr;
  const int32_t* kept_col;
  const int32_t* kept_cnt;
  const int32_t* group_mode;  // [BH] grouping mode per (b, h), or null (mode 0)
  QGroup grp;
  long long nnz;
  int S, Sb, BH;
  int n_tiles;        // query-row tiles per (b, h) (dense) / grid width (sparse)
  float scale_log2;   // softmax_scale * log2(e)
  int spin_limit;     // polls before a bounded wait gives up (>= 1)
};

struct GroupCostParams {
  const int32_t* row_ptr;
  const int32_t* kept_col;
  const int32_t* kept_cnt;
  uint32_t* totals;   // [BH][kGroupModes] kept-list union sizes
  int32_t* group_mode;
  QGroup grp;
  long long nnz;
  int BH, gmax;
};

// N_f limit of the token-level and decay-state selectors (per-frame tables in
// LDS); their own declarations are in token.h and below.
constexpr int kMaxTokenFrames = 64;

// Ordered compaction of one flag per candidate entry into kept lists written
// for every head: flags of batch element b at flags + b * flag_stride
// (flag_stride 0: one mask for all batch elements).
struct FlagCompact {
  const int32_t* row_ptr;
  const int32_t* cols;
  const unsigned char* flags;
  long long flag_stride;
  long long nnz;
  int Sb, H;
  int32_t* kept_col;
  int32_t* kept_cnt;
};
hipError_t launch_flag_compact(const FlagCompact& c, int B, hipStream_t stream);

// Decay-state static-ratio selection ([DR] §3.2 Eq. 8): per frame pair state of
// the sample's threshold search.
struct StaticState {
  uint32_t active;    // 1: t > 1 and t mod sf(t) = 0 (a sampled frame pair)
  uint32_t w;         // window w(t), clamped to N_t
  uint32_t n, k;      // |P(i, j)| and the number of pairs kept
  uint32_t rank;      // rank (1-based) of the k-th key within the current group
  uint32_t group;     // keys agreeing with the resolved prefix
  uint32_t xpre;      // resolved bits of the threshold word
  uint32_t ppre;      // resolved bits of the position cut (ties of the word only)
  uint32_t pos_mode;  // 1: the word ties and positions are being resolved
  uint32_t pcut;      // inclusive position cut among pairs whose word equals xpre
  uint32_t pad[2];
};

struct StaticParams {
  const int32_t* row_ptr;
  const int32_t* cols;
  long long nnz;
  int S, Sb, Nf, Nt, Bs, L0;
  double gamma, lambda, theta_c, theta_m, rho_near, rho_far;
  uint32_t seed_lo, seed_hi;
  StaticState* state;     // [Nf * Nf]
  uint32_t* hist;         // [Nf * Nf][2048]
  unsigned char* flags;   // [nnz]
};
constexpr int kStaticBins = 2048;
hipError_t launch_static_select(const StaticParams& p, hipStream_t stream);

// Proxy-task error sums ([DR] App. C.4 Eq. 22 through a random probe).
constexpr int kProxyPartials = 1024;   // workgroups of the first pass (one float64 triple each)
struct ProxyParams {
  const uint16_t* ref;    // bf16 [n], 16-byte aligned
  const uint16_t* test;   // bf16 [n], 16-byte aligned
  long long n;
  const int32_t* kept_cnt;
  long long n_cnt;
  double* partial;        // [kProxyPartials][3]
  double* out;            // [3], or [6] with the loss terms
  // Eq. 22 terms (with_loss != 0): out[3] = out[0] / out[1] (normalised
  // error), out[4] = 1 - out[2] / total_blocks (sparsity), out[5] = out[3] +
  // alpha * max(0, target - out[4])
  int with_loss;
  long long total_blocks;
  double alpha, target;
};
hipError_t launch_proxy_error(const ProxyParams& p, hipStream_t stream);

hipError_t launch_candidates(const CandParams& p, int32_t* row_ptr, int32_t* cols, long long cap,
                             hipStream_t stream);
hipError_t launch_pool(const PoolParams& p, hipStream_t stream);
size_t tile_desc_bytes(int Sb);
TileDesc tile_desc_at(void* base, int Sb);
hipError_t launch_tile_desc(const ScoreParams& p, hipStream_t stream);
hipError_t launch_scores(const ScoreParams& p, int B, hipStream_t stream);
hipError_t launch_select(const SelectParams& p, int B, hipStream_t stream);
hipError_t launch_sparse_attn(const AttnParams& p, int D, int Bs, hipStream_t stream);
hipError_t launch_dense_attn(const AttnParams& p, int D, hipStream_t stream);
hipError_t launch_group_choice(const GroupCostParams& p, hipStream_t stream);
// Library-held totals of dr_query_groups_noalloc: up to kGroupScratchBH (b, h)
// pairs; the device address of the current device's array.
constexpr int kGroupScratchBH = 65535;
hipError_t group_scratch(uint32_t** out);

}  // namespace dr
