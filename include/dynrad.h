/*
 * dynrad.h -- C ABI of the DynamicRad block-sparse attention hot path for
 * AMD Instinct MI355X (gfx950).
 *
 * Method: "DynamicRad: Content-Adaptive Sparse Attention for Long Video
 * Diffusion" (arXiv 2604.20470), cited below as [DR].
 *
 * The path, one video-DiT self-attention layer at inference:
 *   1. dr_build_candidates  radial block-candidate set ([DR] §3.1, Eqs. 1-7 and
 *                           "Density control within blocks"), content-free.
 *   2. dr_score_select      mean-pooled block scores and dual-mode selection
 *                           ([DR] §3.2: static-ratio / dynamic-threshold).
 *      dr_token_select      the paper's token-level dynamic-threshold selector
 *                           ([DR] §3.2 Eqs. 9-11, Algorithm 1).
 *      dr_static_select     the paper's decay-state static-ratio selector
 *                           ([DR] §3.2 Eq. 8, Algorithm 1), content-free.
 *   3. dr_sparse_attn       flash-style forward attention over the kept KV
 *                           blocks only ([DR] §3.3, Eq. 13 with eps -> 0);
 *      dr_query_groups,     the same with the query blocks grouped so that a
 *      dr_sparse_attn_grouped  workgroup's kept lists overlap most.
 *   dr_attn                 dense forward attention, the speedup denominator
 *                           ([DR] App. A, Eq. 16).
 *   dr_proxy_error          error sums of the proxy-task objective ([DR]
 *                           App. C.4, Eq. 22) from dense and sparse outputs.
 *
 * Conventions shared by every entry point:
 *  - Tensors are [B, H, S, D] row-major and contiguous, bfloat16 (raw 16-bit
 *    patterns), in device memory. S = N_f * N_t tokens, frame-major, raster
 *    order within a frame. Blocks are B_s consecutive tokens; block a holds
 *    tokens [a*B_s, min((a+1)*B_s, S)). S_b = ceil(S / B_s). Tokens >= S are
 *    padding: never attended, never pooled, never written.
 *  - All device buffers are allocated by the caller. The library allocates
 *    nothing. State kept across calls: a thread-local error message, the
 *    process-wide poll limit of the bounded waits (dr_set_wait_limit) and, on
 *    each device, a word of flags of waits that gave up (dr_wait_report).
 *  - Tensor inputs (q, k, v) must hold finite values; NaN or infinity in q or k
 *    makes the outputs of the calls that read them unspecified.
 *  - Calls are asynchronous on the given HIP stream (NULL = default stream);
 *    inputs must stay valid until the stream passes the call. Only
 *    dr_build_candidates synchronises (to report the candidate count).
 *  - Arguments are validated before any launch; an invalid call launches
 *    nothing. No entry point aborts or throws. dr_last_error() describes the
 *    most recent failure on the calling thread.
 *  - Limits: head_dim in {64, 128}; block_size in {32, 64, 128}; S_b <= 16384;
 *    N_f <= 4096; batch * heads * nnz < 2^31.
 */
#ifndef DYNRAD_H
#define DYNRAD_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dr_status {
  DR_OK = 0,
  DR_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, value out of range */
  DR_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim / block_size / size limits */
  DR_ERR_CAPACITY = 3,    /* output capacity below the required size */
  DR_ERR_HIP = 4,         /* a HIP launch or runtime call failed */
  DR_ERR_WAIT = 5         /* dr_wait_report: a bounded wait of a ring kernel gave up */
} dr_status;

/* Radial candidate configuration ([DR] §3.1; parameter vector x of §3.4 / C.4). */
typedef struct dr_radial_cfg {
  int32_t num_frames;       /* N_f >= 1                                              */
  int32_t tokens_per_frame; /* N_t >= 1 (spatial tokens of one latent frame)         */
  int32_t block_size;       /* B_s: 32, 64 or 128 ([DR] Table 4)                     */
  int32_t reserved;         /* must be 0                                             */
  double gamma;             /* decay factor of Eq. 2, > 0                            */
  double lambda;            /* long-range factor of Eq. 4, >= 0                      */
  double theta_c;           /* column density threshold, in [0, 1]                   */
  double theta_m;           /* mask (block activation) threshold, in [0, 1]          */
} dr_radial_cfg;

typedef struct dr_dims {
  int32_t batch;    /* B >= 1                */
  int32_t heads;    /* H >= 1                */
  int32_t head_dim; /* D: 64 or 128          */
  int32_t reserved; /* must be 0             */
} dr_dims;

typedef enum dr_mode {
  DR_STATIC_RATIO = 0,     /* [DR] §3.2 "static_ratio"     */
  DR_DYNAMIC_THRESHOLD = 1 /* [DR] §3.2 "dynamic_threshold" */
} dr_mode;

typedef struct dr_select_cfg {
  int32_t mode;        /* dr_mode                                                        */
  int32_t score_heads; /* 0: one mask per head; g > 0: scores averaged over heads 0..g-1
                          and one mask shared by every head ([DR] App. B, Eq. 19)         */
  double ratio;        /* static: keep max(1, ceil(ratio * n - 1e-9)) of n, ratio in (0,1] */
  double tau;          /* dynamic: cumulative softmax mass to reach, tau in (0, 1]       */
} dr_select_cfg;

/* Number of blocks S_b = ceil(N_f * N_t / B_s) for a valid configuration, else
 * a negative dr_status. Host only. */
int64_t dr_num_blocks(const dr_radial_cfg* cfg);

/* Per-distance table of [DR] §3.1 Eqs. 1-5, the table the candidate kernel uses:
 * w[t] (window width, Eq. 3) and sf[t] (split stride, Eq. 5) for t in [0, N_f).
 * t = 0: w = N_t, sf = 1 (dense). t >= 1: L0 = next power of two >= N_t,
 * B(t) = floor(log2 t) + 1, L = L0 / 2^B(t) * gamma, w = N_t if t == 1 else
 * max(B_s, floor(L + 1/2)); sf = max(1, floor(B_s / (L0 / 2^B(t) * lambda + 1e-6))).
 * Evaluated in IEEE double, no contraction. w and sf are host arrays of
 * num_frames int32 (windows above 2^30 saturate there; any w >= N_t - 1 admits
 * every spatial pair). Host only. */
dr_status dr_distance_table(const dr_radial_cfg* cfg, int32_t* w, int32_t* sf);

/* Candidate block set ([DR] §3.1 Eqs. 6-7, "Density control within blocks").
 * Token pair (q, k) with frame distance t and local indices u_q, u_k is a
 * candidate iff t mod sf(t) == 0 and |u_q - u_k| <= w(t). For block pair
 * (a, b): a key token of b is active iff (query tokens of a paired with it) /
 * (query tokens of a) > theta_c; (a, b) is a candidate iff (active key tokens)
 * / (key tokens of b) > theta_m. Padding tokens count nowhere.
 * Output, device memory, CSR over query blocks:
 *   row_ptr [S_b + 1] int32: row a's candidates are cols[row_ptr[a] .. row_ptr[a+1]);
 *   cols    [cap]     int32: key-block indices, strictly ascending within a row.
 * nnz (host pointer): if non-NULL, the call synchronises the stream and stores
 * the candidate count; if it exceeds cap, returns DR_ERR_CAPACITY (cols holds
 * the first cap entries; call again with cap >= *nnz). If NULL, the call is
 * asynchronous, writes past cap are dropped and the count is row_ptr[S_b]. */
dr_status dr_build_candidates(const dr_radial_cfg* cfg, int32_t* row_ptr, int32_t* cols,
                              int64_t cap, int64_t* nnz, hipStream_t stream);

/* Device workspace (bytes) dr_score_select needs: pooled Q and K means (float32,
 * [B, Hs, S_b, D] each, Hs = H or score_heads), the score buffer (float32,
 * [B * Hm * nnz], Hm = H or 1) and a head-independent map of the candidate
 * tiles (about 260 * ceil(S_b / 32)^2 bytes). Host only. */
dr_status dr_score_select_workspace(const dr_dims* dims, const dr_radial_cfg* cfg,
                                    const dr_select_cfg* sel, int64_t nnz, size_t* bytes);

/* Block scoring and dual-mode selection ([DR] §3.2, block form).
 *  1. Block means of Q and K over valid tokens (float32).
 *  2. Scores on the candidate entries: s(a, c) = Qbar_a . Kbar_c / sqrt(D)
 *     (block form of [DR] Eq. 9); with score_heads = g > 0 the mean over heads
 *     0..g-1 ([DR] Eq. 19), and the mask is shared by every head.
 *  3. Per query block with n candidates, order by (score desc, key index asc):
 *     static  keeps the first k = max(1, ceil(ratio * n - 1e-9));
 *     dynamic keeps the shortest prefix whose softmax mass (softmax of the raw
 *     scores over the n candidates) reaches tau, at least one ([DR] §3.2
 *     safeguard (ii)); tau >= 1 keeps all.
 * Inputs: q, k bf16 [B, H, S, D] (device); row_ptr, cols from dr_build_candidates.
 * Outputs (device):
 *   kept_col [B * H * nnz] int32: the kept list of (b, h, a) starts at
 *       (b * H + h) * nnz + row_ptr[a], ascending key-block indices;
 *   kept_cnt [B * H * S_b] int32: its length, at (b * H + h) * S_b + a.
 *   scores_out: NULL, or float32 [B * Hm * nnz] receiving the scores in CSR order.
 * ws / ws_bytes: device workspace of at least dr_score_select_workspace bytes. */
dr_status dr_score_select(const dr_dims* dims, const dr_radial_cfg* cfg, const dr_select_cfg* sel,
                          const void* q, const void* k, const int32_t* row_ptr, const int32_t* cols,
                          int64_t nnz, int32_t* kept_col, int32_t* kept_cnt, float* scores_out,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* Token-level dynamic-threshold selection: the selector of [DR] §3.2
 * "Dynamic-threshold mode" (Eqs. 9-11, "Global thresholding with safeguards",
 * Algorithm 1), aggregated to blocks by the density control of §3.1.
 * For every frame pair (i, j), t = |i - j|:
 *   - t mod sf(t) != 0: no pair (Eq. 6);
 *   - t <= 1: every pair of P(i, j) is selected (tau = -inf, Eq. 11; t = 0 is
 *     dense attention);
 *   - otherwise s(u, v) = (1/H_f) sum_{h < H_f} Q_u^h . K_v^h / sqrt(d_k) (Eq. 9)
 *     on P(i, j) = {|u - v| <= w(t)} (Eq. 7); z = (s - mu_ij) / (sigma_ij + eps)
 *     with mu, sigma the mean and population standard deviation of s over
 *     P(i, j) (Eq. 10); a pair is selected iff z >= tau(t), tau = tau_near if
 *     L(t) = L0 / 2^B(t) * gamma >= B_s, else tau_far (Eq. 11); if no pair of
 *     P(i, j) is selected, its highest-scoring pair is (safeguard (ii); ties:
 *     the first in (u, v) order).
 * Block pair (a, b) is kept iff, over all frame pairs it spans, the share of
 * b's key tokens whose selected share of a's query tokens exceeds theta_c
 * itself exceeds theta_m (cfg->theta_c, cfg->theta_m). The heads 0..H_f-1 of
 * each batch element decide one mask, written for every head.
 * Inputs: q, k bf16 [B, H, S, D]; row_ptr, cols from dr_build_candidates with
 * the same cfg (the kept set is always a subset of the candidate set).
 * Outputs: kept_col / kept_cnt in the layout of dr_score_select.
 * Limits: tokens_per_frame in [32, 65535], num_frames <= 64, fused_heads in
 * {1, 2} (<= heads), eps > 0, tau_near and tau_far not NaN (+-inf allowed).
 * Deterministic: statistics are merged in a fixed order (no float atomics).
 * At block size 32 and 64 most block decisions are fixed from per-column sums
 * of the statistics pass (exactly: the same flags as computing every tile);
 * the environment variable DR_TOKEN_RING_MARK=1, read at each call, makes the
 * library compute every tile instead (a reference path for tests). */
typedef struct dr_token_cfg {
  int32_t fused_heads;  /* H_f: 1 or 2 ([DR] Table 4: 2)                   */
  int32_t reserved;     /* must be 0                                        */
  double tau_near;      /* tau_1, near_frame_thresh (Eq. 11)                */
  double tau_far;       /* tau_2, far_frame_thresh                          */
  double eps;           /* epsilon of Eq. 10, > 0                           */
} dr_token_cfg;

/* Device workspace (bytes) of dr_token_select. Host only. */
dr_status dr_token_select_workspace(const dr_dims* dims, const dr_radial_cfg* cfg, const dr_token_cfg* tok,
                                    int64_t nnz, size_t* bytes);

dr_status dr_token_select(const dr_dims* dims, const dr_radial_cfg* cfg, const dr_token_cfg* tok,
                          const void* q, const void* k, const int32_t* row_ptr, const int32_t* cols,
                          int64_t nnz, int32_t* kept_col, int32_t* kept_cnt, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* Decay-state static-ratio selection: the selector of [DR] §3.2 "Static-ratio
 * mode" (Eq. 8, Algorithm 1), aggregated to blocks by the density control of
 * §3.1. It reads no tensor: the mask depends on cfg, rho and the seed only, so
 * it is built once and reused for every layer and step.
 * For every frame pair (i, j), t = |i - j|:
 *   - t mod sf(t) != 0: no pair (Eq. 6);
 *   - t <= 1: every pair of P(i, j) is selected (rho = 1; t = 0 is dense);
 *   - otherwise k = max(1, floor(|P(i, j)| * rho + 1e-9)) (float64) pairs of
 *     P(i, j) = {|u - v| <= w(t)} (Eq. 7), rho = rho_near if
 *     L(t) = L0 / 2^B(t) * gamma >= B_s else rho_far (Eq. 8), drawn uniformly
 *     with the seed: pair (u, v) gets the 32-bit output word (v mod 4) of
 *     Philox4x32-10 (Salmon et al., "Parallel Random Numbers: As Easy as 1, 2,
 *     3", SC 2011) at counter (u, floor(v / 4), i, j) under the key
 *     (seed mod 2^32, seed div 2^32), and the k pairs with the smallest
 *     (word, u * N_t + v) are selected (a uniformly random k-subset).
 * Block pair (a, b) is kept iff, over all frame pairs it spans, the share of
 * b's key tokens whose selected share of a's query tokens exceeds theta_c
 * itself exceeds theta_m. The one mask is written for every (b, h) of dims
 * (head_dim is not used; pass batch = heads = 1 for a single copy).
 * Inputs: row_ptr, cols from dr_build_candidates with the same cfg.
 * Outputs: kept_col / kept_cnt in the layout of dr_score_select.
 * Limits: tokens_per_frame in [32, 65535], num_frames <= 64, rho_near and
 * rho_far in [0, 1]. Bit-reproducible (integer work only). */
typedef struct dr_static_cfg {
  double rho_near;   /* rho_1, topk_ratio1: retention for t > 1, L(t) >= B_s (Eq. 8) */
  double rho_far;    /* rho_2, topk_ratio2: retention for t > 1, L(t) <  B_s         */
  uint64_t seed;     /* Philox key: (seed mod 2^32, seed div 2^32)                  */
} dr_static_cfg;

/* Device workspace (bytes) of dr_static_select: 48 + 8192 bytes per ordered
 * frame pair, plus nnz bytes (each part 256-byte aligned). Host only. */
dr_status dr_static_select_workspace(const dr_radial_cfg* cfg, int64_t nnz, size_t* bytes);

dr_status dr_static_select(const dr_dims* dims, const dr_radial_cfg* cfg, const dr_static_cfg* st,
                           const int32_t* row_ptr, const int32_t* cols, int64_t nnz, int32_t* kept_col,
                           int32_t* kept_cnt, void* ws, size_t ws_bytes, hipStream_t stream);

/* Block-sparse forward attention ([DR] §3.3 Eqs. 12-13, eps -> 0): for each
 * (b, h) and query block a, O[rows of a] = softmax(Q K^T * softmax_scale) V over
 * the valid key tokens of the blocks in a's kept list only; online softmax in
 * float32, bf16 products into float32 accumulators, bf16 output.
 * Kept lists use the layout of dr_score_select (any source: a host-built mask
 * uploaded in that layout works). Entries outside [0, S_b) are ignored and
 * duplicates count once; a row with no kept block outputs zeros; a kept count
 * above the row's candidate count is read as the candidate count.
 * q, k, v, out: bf16 [B, H, S, D] device; out must not alias the inputs. */
dr_status dr_sparse_attn(const dr_dims* dims, const dr_radial_cfg* cfg, const void* q,
                         const void* k, const void* v, const int32_t* row_ptr, int64_t nnz,
                         const int32_t* kept_col, const int32_t* kept_cnt, float softmax_scale,
                         void* out, hipStream_t stream);

/* Query-block grouping of the sparse attention (scheduling only). One
 * workgroup computes a group of Q = 256 / B_s query blocks and reads the union
 * of their kept lists ([DR] §3.3: each kept block pair is one tile), so groups
 * whose kept lists overlap read fewer key/value bytes. The workgroup streams
 * that union in an order set by all of its query blocks (round robin over
 * their kept lists by rank), so a grouping changes the order in which a query
 * block's kept blocks are accumulated: outputs of different groupings agree to
 * float32 rounding, and each is bitwise reproducible. Modes:
 *   0: consecutive blocks Q g .. Q g + Q - 1 (the grouping of dr_sparse_attn);
 *   1, 2: blocks in rows, one per frame (row f = blocks [floor(f N_t / B_s),
 *      floor((f + 1) N_t / B_s)), the last row up to S_b); a group is F
 *      consecutive rows by R adjacent columns, (F, R) = (4, 2) and (2, 4) at
 *      B_s = 32, (2, 2) and (4, 1) at 64, (2, 1) at 128 (mode 2 has no group
 *      at 128).
 * Each mode partitions [0, S_b) into groups of at most Q blocks.
 *
 * dr_query_group_table (host only): the blocks of every group of a mode, Q per
 * group in slot order, -1 for an empty slot; returns the entry count (groups
 * times Q) or a negative dr_status. table = NULL only returns the count; else
 * cap must reach it. */
int64_t dr_query_group_table(const dr_radial_cfg* cfg, int32_t mode, int32_t* table, int64_t cap);

/* Device workspace (bytes) of dr_query_groups: 12 bytes per (b, h), rounded up
 * to 256. Host only. */
dr_status dr_query_groups_workspace(const dr_dims* dims, size_t* bytes);

/* Per (b, h), the grouping mode whose groups' kept-list unions have the
 * smallest estimated total size: the union sizes of groups 0, 4, 8, ... of a
 * mode, summed and scaled by (groups of the mode) / (groups measured); ties go
 * to the lower mode. Kept lists in the layout of dr_score_select. Integer work
 * (compared by cross-multiplication), deterministic.
 * group_mode: device int32 [B * H] (output); ws: device workspace of at least
 * dr_query_groups_workspace bytes; B * H <= 65535. */
dr_status dr_query_groups(const dr_dims* dims, const dr_radial_cfg* cfg, const int32_t* row_ptr,
                          int64_t nnz, const int32_t* kept_col, const int32_t* kept_cnt,
                          int32_t* group_mode, void* ws, size_t ws_bytes, hipStream_t stream);

/* dr_query_groups for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * computation and outputs, with the union totals held in a scratch array the
 * library keeps in each GPU's memory for the life of the process (12 bytes per
 * (b, h), 768 KiB per GPU for the limit B * H <= 65535; its device address is
 * taken once per device, on the first call with that device current). It
 * allocates nothing and calls no allocating routine. Every call on a GPU uses
 * that GPU's one array: calls that overlap on one GPU (other streams, other
 * threads) race and must not be issued; each call clears what it uses before
 * use. `stream` must belong to the current device. */
dr_status dr_query_groups_noalloc(const dr_dims* dims, const dr_radial_cfg* cfg, const int32_t* row_ptr,
                                  int64_t nnz, const int32_t* kept_col, const int32_t* kept_cnt,
                                  int32_t* group_mode, hipStream_t stream);

/* dr_sparse_attn with the query blocks of (b, h) grouped by mode
 * group_mode[b * H + h] (device int32 [B * H], non-NULL; a value that is not a
 * mode with groups at this B_s means mode 0). Same results as dr_sparse_attn up
 * to the order of accumulation. */
dr_status dr_sparse_attn_grouped(const dr_dims* dims, const dr_radial_cfg* cfg, const void* q,
                                 const void* k, const void* v, const int32_t* row_ptr, int64_t nnz,
                                 const int32_t* kept_col, const int32_t* kept_cnt,
                                 const int32_t* group_mode, float softmax_scale, void* out,
                                 hipStream_t stream);

/* Dense forward attention over all seq_len keys (bidirectional), the baseline
 * of [DR] App. A Eq. 16 / Table 5 "Dense". Same numerics and layouts as
 * dr_sparse_attn; seq_len >= 1. */
dr_status dr_attn(const dr_dims* dims, int32_t seq_len, const void* q, const void* k,
                  const void* v, float softmax_scale, void* out, hipStream_t stream);

/* Proxy-task error sums ([DR] App. C.4 "Optimization Objective", Eq. 22).
 * Eq. 22 compares the dense attention matrix A with the kept-block one A'.
 * With o_ref = dr_attn(Q, K, Z) and o_test = dr_sparse_attn(Q, K, Z, mask) for
 * a probe Z of independent N(0, 1) entries, E ||o_test - o_ref||^2 =
 * D ||A' - A||_F^2 and E ||o_ref||^2 = D ||A||_F^2, so
 *   out[0] = sum_i (o_test[i] - o_ref[i])^2     (i < n, bf16 inputs)
 *   out[1] = sum_i o_ref[i]^2
 *   out[2] = sum_j kept_cnt[j]                  (j < n_cnt; 0 if kept_cnt is NULL)
 * give the normalised error out[0] / out[1] and the sparsity
 * 1 - out[2] / (B * H * S_b^2); the loss is that error plus
 * alpha * max(0, target - sparsity) (alpha = 10, target = 0.8 in [DR]).
 * Sums in float64, fixed summation order (bit-reproducible).
 * o_ref, o_test: device, 16-byte aligned; out: device, 3 doubles; ws: device
 * workspace of at least DR_PROXY_WS_BYTES bytes. */
#define DR_PROXY_WS_BYTES 24576
dr_status dr_proxy_error(const void* o_ref, const void* o_test, int64_t n, const int32_t* kept_cnt, int64_t n_cnt,
                         double* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* The proxy-task objective of [DR] App. C.4 Eq. 22 in one call: the sums of
 * dr_proxy_error in out[0..2], then
 *   out[3] = out[0] / out[1]                          normalised error
 *   out[4] = 1 - out[2] / total_blocks                sparsity (total_blocks =
 *                                                     B * H * S_b^2, all block pairs)
 *   out[5] = out[3] + alpha * max(0, target - out[4]) the loss ([DR]: alpha = 10,
 *                                                     target = 0.8)
 * out: device, 6 doubles; total_blocks >= 1; alpha finite and >= 0; target
 * finite. out[1] = 0 (an all-zero o_ref) gives the IEEE quotient (inf or NaN).
 * Other arguments as dr_proxy_error. */
dr_status dr_proxy_loss(const void* o_ref, const void* o_test, int64_t n, const int32_t* kept_cnt, int64_t n_cnt,
                        int64_t total_blocks, double alpha, double target, double* out, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* Bounded waits. The kernels of dr_sparse_attn, dr_sparse_attn_grouped,
 * dr_attn and dr_token_select pass data between wavefronts through LDS rings
 * ([DR] §3.3: each kept tile is streamed once per workgroup); every wait in
 * them polls a bounded number of times. A wave whose wait gives up (the
 * protocol never needs it) sets a flag on its device and goes on, so the
 * kernel still exits, but the outputs of that call are not valid.
 *
 * dr_wait_report: synchronises `stream`, then reads and clears the flags of
 * the current device: bit 0 (1) an attention loader refilled a slot before it
 * was free, bit 1 (2) an attention compute wave read a unit before it was
 * published, bit 2 (4) a token-selection wave read a key block before it was
 * published. Stores them in *flags (host) and returns DR_ERR_WAIT if any is
 * set, else DR_OK. Calls still running on other streams may set flags later.
 *
 * dr_set_wait_limit: the number of polls after which every bounded wait of
 * later calls (on any device, any thread) gives up; 0 restores the default
 * 2^26 (seconds of waiting). For tests of this report: a tiny limit makes
 * waits give up on purpose while every kernel still exits normally. */
dr_status dr_wait_report(hipStream_t stream, uint32_t* flags);
dr_status dr_set_wait_limit(int64_t polls);

/* Static description of a status code. */
const char* dr_status_string(dr_status status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* dr_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DYNRAD_H */
