// C ABI of the DynamicRad hot path (include/dynrad.h): argument validation,
// the host per-distance table, workspace layout and kernel launches.
// Every check runs before any HIP call, so an invalid call touches no device.
#include <math.h>
#include <algorithm>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <string>

#include "../../include/dynrad.h"
#include "dr_internal.h"
#include "token.h"

namespace {

thread_local std::string g_last_error;

// Polls before a bounded wait of the ring kernels gives up (dr_set_wait_limit).
std::atomic<int> g_wait_limit{dr::kDefaultSpinLimit};

dr_status fail(dr_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

dr_status ok() {
  g_last_error.clear();
  return DR_OK;
}

dr_status hip_fail(hipError_t e, const char* what) {
  return fail(DR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool finite(double x) { return isfinite(x) != 0; }

struct Layout {
  long long S;
  int Sb;
};

dr_status check_radial(const dr_radial_cfg* c, Layout* out) {
  if (!c) return fail(DR_ERR_INVALID_ARG, "radial config is NULL");
  if (c->num_frames < 1 || c->tokens_per_frame < 1 || c->block_size < 1)
    return fail(DR_ERR_INVALID_ARG, "num_frames, tokens_per_frame and block_size must be >= 1");
  if (c->reserved != 0) return fail(DR_ERR_INVALID_ARG, "radial config reserved field must be 0");
  if (!finite(c->gamma) || c->gamma <= 0.0) return fail(DR_ERR_INVALID_ARG, "gamma must be finite and > 0");
  if (!finite(c->lambda) || c->lambda < 0.0) return fail(DR_ERR_INVALID_ARG, "lambda must be finite and >= 0");
  if (!finite(c->theta_c) || c->theta_c < 0.0 || c->theta_c > 1.0)
    return fail(DR_ERR_INVALID_ARG, "theta_c must be in [0, 1]");
  if (!finite(c->theta_m) || c->theta_m < 0.0 || c->theta_m > 1.0)
    return fail(DR_ERR_INVALID_ARG, "theta_m must be in [0, 1]");
  if (c->block_size != 32 && c->block_size != 64 && c->block_size != 128)
    return fail(DR_ERR_UNSUPPORTED, "block_size %d not built (32, 64 or 128)", c->block_size);
  if (c->num_frames > dr::kMaxFrames)
    return fail(DR_ERR_UNSUPPORTED, "num_frames %d above the limit %d", c->num_frames, dr::kMaxFrames);
  const long long S = (long long)c->num_frames * c->tokens_per_frame;
  const long long Sb = (S + c->block_size - 1) / c->block_size;
  if (Sb > dr::kMaxBlocks)
    return fail(DR_ERR_UNSUPPORTED, "S_b = %lld blocks above the limit %d", Sb, dr::kMaxBlocks);
  if (out) {
    out->S = S;
    out->Sb = (int)Sb;
  }
  return DR_OK;
}

dr_status check_dims(const dr_dims* d) {
  if (!d) return fail(DR_ERR_INVALID_ARG, "dims is NULL");
  if (d->batch < 1 || d->heads < 1 || d->head_dim < 1)
    return fail(DR_ERR_INVALID_ARG, "batch, heads and head_dim must be >= 1");
  if (d->reserved != 0) return fail(DR_ERR_INVALID_ARG, "dims reserved field must be 0");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(DR_ERR_UNSUPPORTED, "head_dim %d not built (64 or 128)", d->head_dim);
  if ((long long)d->batch * d->heads > 65535)
    return fail(DR_ERR_UNSUPPORTED, "batch * heads above 65535");
  return DR_OK;
}

dr_status check_select(const dr_select_cfg* s, const dr_dims* d) {
  if (!s) return fail(DR_ERR_INVALID_ARG, "select config is NULL");
  if (s->mode != DR_STATIC_RATIO && s->mode != DR_DYNAMIC_THRESHOLD)
    return fail(DR_ERR_INVALID_ARG, "mode %d is neither static_ratio (0) nor dynamic_threshold (1)", s->mode);
  if (s->score_heads < 0 || s->score_heads > d->heads)
    return fail(DR_ERR_INVALID_ARG, "score_heads %d outside [0, heads]", s->score_heads);
  if (s->mode == DR_STATIC_RATIO && (!finite(s->ratio) || s->ratio <= 0.0 || s->ratio > 1.0))
    return fail(DR_ERR_INVALID_ARG, "ratio must be in (0, 1]");
  if (s->mode == DR_DYNAMIC_THRESHOLD && (!finite(s->tau) || s->tau <= 0.0 || s->tau > 1.0))
    return fail(DR_ERR_INVALID_ARG, "tau must be in (0, 1]");
  return DR_OK;
}

dr_status check_nnz(long long nnz, int Sb, const dr_dims* d) {
  if (nnz < 1 || nnz > (long long)Sb * Sb)
    return fail(DR_ERR_INVALID_ARG, "nnz %lld outside [1, S_b^2]", nnz);
  if ((long long)d->batch * d->heads * nnz >= (1LL << 31))
    return fail(DR_ERR_UNSUPPORTED, "batch * heads * nnz reaches 2^31");
  return DR_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t qbar, kbar, scores, tiles, total;
  int Hp, Hm, g;
};

WsLayout ws_layout(const dr_dims* d, int Sb, const dr_select_cfg* s, long long nnz) {
  WsLayout w;
  w.g = s->score_heads > 0 ? s->score_heads : 1;
  w.Hp = s->score_heads > 0 ? s->score_heads : d->heads;
  w.Hm = s->score_heads > 0 ? 1 : d->heads;
  const size_t pooled = align256((size_t)d->batch * w.Hp * Sb * d->head_dim * sizeof(float));
  w.qbar = 0;
  w.kbar = pooled;
  w.scores = 2 * pooled;
  w.tiles = w.scores + align256((size_t)d->batch * w.Hm * nnz * sizeof(float));
  w.total = w.tiles + dr::tile_desc_bytes(Sb);
  return w;
}

struct TokWs {
  size_t part, thr, fmax, fn, served, flags, colsum, und, total;
  int n_wg, FR;
  bool decide;   // B_s = 32: column sums and the decision pass
};

TokWs tok_ws(const dr_dims* d, const dr_radial_cfg* c, int Sb, long long S, long long nnz) {
  TokWs w;
  const int Nf = c->num_frames;
  w.n_wg = (int)((S + 255) / 256);
  w.FR = 255 / c->tokens_per_frame + 2;
  const size_t fpairs = (size_t)d->batch * Nf * Nf;
  size_t off = 0;
  w.part = off;
  off = align256(off + (size_t)d->batch * w.n_wg * dr::kTokSplit * w.FR * Nf * sizeof(dr::TokStat));
  w.thr = off;
  off = align256(off + fpairs * sizeof(float));
  w.fmax = off;
  off = align256(off + fpairs * sizeof(unsigned long long));
  w.fn = off;
  off = align256(off + fpairs * sizeof(double));
  w.served = off;
  off = align256(off + fpairs * sizeof(int));
  w.flags = off;
  off = align256(off + (size_t)d->batch * nnz);
  w.decide = c->block_size <= 64;   // one 32 x 32 tile's column sums per sub-tile pair
  const size_t tiles = w.decide ? (size_t)(c->block_size / 32) * (c->block_size / 32) : 0;
  w.colsum = off;
  if (w.decide) off = align256(off + (size_t)d->batch * nnz * tiles * 32 * 2 * sizeof(float));
  w.und = off;
  if (w.decide) off = align256(off + (size_t)d->batch * nnz);
  w.total = off;
  (void)Sb;
  return w;
}

dr_status check_token(const dr_token_cfg* t, const dr_dims* d, const dr_radial_cfg* c, int Sb) {
  if (!t) return fail(DR_ERR_INVALID_ARG, "token config is NULL");
  if (t->reserved != 0) return fail(DR_ERR_INVALID_ARG, "token config reserved field must be 0");
  if (t->fused_heads < 1 || t->fused_heads > d->heads)
    return fail(DR_ERR_INVALID_ARG, "fused_heads %d outside [1, heads]", t->fused_heads);
  if (t->fused_heads > 2) return fail(DR_ERR_UNSUPPORTED, "fused_heads %d not built (1 or 2)", t->fused_heads);
  if (isnan(t->tau_near) || isnan(t->tau_far)) return fail(DR_ERR_INVALID_ARG, "tau_near / tau_far is NaN");
  if (!finite(t->eps) || t->eps <= 0.0) return fail(DR_ERR_INVALID_ARG, "eps must be finite and > 0");
  if (c->tokens_per_frame < 32 || c->tokens_per_frame > 65535)
    return fail(DR_ERR_UNSUPPORTED, "token-level selection needs tokens_per_frame in [32, 65535]");
  if (c->num_frames > dr::kMaxTokenFrames)
    return fail(DR_ERR_UNSUPPORTED, "token-level selection needs num_frames <= %d", dr::kMaxTokenFrames);
  const size_t lds = dr::token_lds_bytes(d->head_dim, c->block_size, t->fused_heads, Sb, c->num_frames,
                                         255 / c->tokens_per_frame + 2);
  if (lds > 160 * 1024) return fail(DR_ERR_UNSUPPORTED, "token-level selection needs %zu bytes of LDS", lds);
  return DR_OK;
}

}  // namespace

extern "C" {

int64_t dr_num_blocks(const dr_radial_cfg* cfg) {
  Layout L;
  const dr_status st = check_radial(cfg, &L);
  if (st != DR_OK) return -(int64_t)st;
  ok();
  return L.Sb;
}

dr_status dr_distance_table(const dr_radial_cfg* cfg, int32_t* w, int32_t* sf) {
  dr_status st = check_radial(cfg, nullptr);
  if (st != DR_OK) return st;
  if (!w || !sf) return fail(DR_ERR_INVALID_ARG, "w and sf must be non-NULL");
  const int L0 = dr::base_span(cfg->tokens_per_frame);
  for (int t = 0; t < cfg->num_frames; ++t) {
    int ww, ss;
    dr::table_entry(t, cfg->tokens_per_frame, cfg->block_size, L0, cfg->gamma, cfg->lambda, &ww, &ss);
    w[t] = ww;
    sf[t] = ss;
  }
  return ok();
}

dr_status dr_build_candidates(const dr_radial_cfg* cfg, int32_t* row_ptr, int32_t* cols, int64_t cap,
                              int64_t* nnz, hipStream_t stream) {
  Layout L;
  dr_status st = check_radial(cfg, &L);
  if (st != DR_OK) return st;
  if (!row_ptr || !cols) return fail(DR_ERR_INVALID_ARG, "row_ptr and cols must be non-NULL");
  if (cap < 1) return fail(DR_ERR_INVALID_ARG, "cap must be >= 1");
  dr::CandParams p;
  p.Nf = cfg->num_frames;
  p.Nt = cfg->tokens_per_frame;
  p.Bs = cfg->block_size;
  p.S = (int)L.S;
  p.Sb = L.Sb;
  p.L0 = dr::base_span(p.Nt);
  p.gamma = cfg->gamma;
  p.lambda = cfg->lambda;
  p.theta_c = cfg->theta_c;
  p.theta_m = cfg->theta_m;
  hipError_t e = dr::launch_candidates(p, row_ptr, cols, cap, stream);
  if (e != hipSuccess) return hip_fail(e, "candidate kernels");
  if (nnz) {
    int32_t total = 0;
    e = hipMemcpyAsync(&total, row_ptr + L.Sb, sizeof(int32_t), hipMemcpyDeviceToHost, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(nnz)");
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    *nnz = total;
    if (total > cap)
      return fail(DR_ERR_CAPACITY, "candidate count %d exceeds cap %lld", total, (long long)cap);
  }
  return ok();
}

dr_status dr_score_select_workspace(const dr_dims* dims, const dr_radial_cfg* cfg, const dr_select_cfg* sel,
                                    int64_t nnz, size_t* bytes) {
  Layout L;
  dr_status st = check_radial(cfg, &L);
  if (st != DR_OK) return st;
  if ((st = check_dims(dims)) != DR_OK) return st;
  if ((st = check_select(sel, dims)) != DR_OK) return st;
  if ((st = check_nnz(nnz, L.Sb, dims)) != DR_OK) return st;
  if (!bytes) return fail(DR_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = ws_layout(dims, L.Sb, sel, nnz).total;
  return ok();
}

dr_status dr_score_select(const dr_dims* dims, const dr_radial_cfg* cfg, const dr_select_cfg* sel,
                          const void* q, const void* k, const int32_t* row_ptr, const int32_t* cols,
                          int64_t nnz, int32_t* kept_col, int32_t* kept_cnt, float* scores_out, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  Layout L;
  dr_status st = check_radial(cfg, &L);
  if (st != DR_OK) return st;
  if ((st = check_dims(dims)) != DR_OK) return st;
  if ((st = check_select(sel, dims)) != DR_OK) return st;
  if ((st = check_nnz(nnz, L.Sb, dims)) != DR_OK) return st;
  if (!q || !k || !row_ptr || !cols || !kept_col || !kept_cnt || !ws)
    return fail(DR_ERR_INVALID_ARG, "q, k, row_ptr, cols, kept_col, kept_cnt and ws must be non-NULL");
  const WsLayout w = ws_layout(dims, L.Sb, sel, nnz);
  if (ws_bytes < w.total)
    return fail(DR_ERR_CAPACITY, "workspace of %zu bytes below the %zu required", ws_bytes, w.total);
  unsigned char* wsb = static_cast<unsigned char*>(ws);
  float* qbar = reinterpret_cast<float*>(wsb + w.qbar);
  float* kbar = reinterpret_cast<float*>(wsb + w.kbar);
  float* scores = scores_out ? scores_out : reinterpret_cast<float*>(wsb + w.scores);

  dr::PoolParams pp;
  pp.q = static_cast<const uint16_t*>(q);
  pp.k = static_cast<const uint16_t*>(k);
  pp.qbar = qbar;
  pp.kbar = kbar;
  pp.B = dims->batch;
  pp.H = dims->heads;
  pp.Hp = w.Hp;
  pp.S = (int)L.S;
  pp.Sb = L.Sb;
  pp.Bs = cfg->block_size;
  pp.D = dims->head_dim;
  hipError_t e = dr::launch_pool(pp, stream);
  if (e != hipSuccess) return hip_fail(e, "pool kernel");

  dr::ScoreParams sp;
  sp.qbar = qbar;
  sp.kbar = kbar;
  sp.row_ptr = row_ptr;
  sp.cols = cols;
  sp.scores = scores;
  sp.nnz = nnz;
  sp.Sb = L.Sb;
  sp.Hp = w.Hp;
  sp.Hm = w.Hm;
  sp.g = w.g;
  sp.D = dims->head_dim;
  sp.scale = (float)(1.0 / (sqrt((double)dims->head_dim) * (double)w.g));
  sp.tiles = dr::tile_desc_at(wsb + w.tiles, L.Sb);
  e = dr::launch_tile_desc(sp, stream);
  if (e != hipSuccess) return hip_fail(e, "tile kernel");
  e = dr::launch_scores(sp, dims->batch, stream);
  if (e != hipSuccess) return hip_fail(e, "score kernel");

  dr::SelectParams xp;
  xp.scores = scores;
  xp.row_ptr = row_ptr;
  xp.cols = cols;
  xp.kept_col = kept_col;
  xp.kept_cnt = kept_cnt;
  xp.nnz = nnz;
  xp.Sb = L.Sb;
  xp.H = dims->heads;
  xp.Hm = w.Hm;
  xp.mode = sel->mode;
  xp.ratio = sel->ratio;
  xp.tau = sel->tau;
  xp.max_row = L.Sb;
  e = dr::launch_select(xp, dims->batch, stream);
  if (e != hipSuccess) return hip_fail(e, "select kernel");
  return ok();
}

static dr_status attn_common(const dr_dims* dims, long long S, const void* q, const void* k, const void* v,
                             float scale, void* out, dr::AttnParams* p) {
  if (!q || !k || !v || !out) return fail(DR_ERR_INVALID_ARG, "q, k, v and out must be non-NULL");
  if (!isfinite(scale)) return fail(DR_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (out == q || out == k || out == v) return fail(DR_ERR_INVALID_ARG, "out must not alias q, k or v");
  if ((long long)dims->batch * dims->heads * S * dims->head_dim >= (1LL << 40))
    return fail(DR_ERR_UNSUPPORTED, "tensor too large");
  p->q = static_cast<const uint16_t*>(q);
  p->k = static_cast<const uint16_t*>(k);
  p->v = static_cast<const uint16_t*>(v);
  p->o = static_cast<uint16_t*>(out);
  p->S = (int)S;
  p->BH = dims->batch * dims->heads;
  p->n_tiles = (int)((S + 255) / 256);
  p->group_mode = nullptr;
  p->grp = dr::QGroup{};
  p->scale_log2 = scale * 1.4426950408889634f;
  p->spin_limit = g_wait_limit.load(std::memory_order_relaxed);
  return DR_OK;
}

dr_status dr_token_select_workspace(const dr_dims* dims, const dr_radial_cfg* cfg, const dr_token_cfg* tok,
                                    int64_t nnz, size_t* bytes) {
  Layout L;
  dr_status st = check_radial(cfg, &L);
  if (st != DR_OK) return st;
  if ((st = check_dims(dims)) != DR_OK) return st;
  if ((st = check_token(tok, dims, cfg, L.Sb)) != DR_OK) return st;
  if ((st = check_nnz(nnz, L.Sb, dims)) != DR_OK) return st;
  if (!bytes) return fail(DR_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = tok_ws(dims, cfg, L.Sb, L.S, nnz).total;
  return ok();
}

dr_status dr_token_select(const dr_dims* dims, const dr_radial_cfg* cfg, const dr_token_cfg* tok, const void* q,
                          const void* k, const int32_t* row_ptr, const int32_t* cols, int64_t nnz,
                          int32_t* kept_col, int32_t* kept_cnt, void* ws, size_t ws_bytes, hipStream_t stream) {
  Layout L;
  dr_status st = check_radial(cfg, &L);
  if (st != DR_OK) return st;
  if ((st = check_dims(dims)) != DR_OK) return st;
  if ((st = check_token(tok, dims, cfg, L.Sb)) != DR_OK) return st;
  if ((st = check_nnz(nnz, L.Sb, dims)) != DR_OK) return st;
  if (!q || !k || !row_ptr || !cols || !kept_col || !kept_cnt || !ws)
    return fail(DR_ERR_INVALID_ARG, "q, k, row_ptr, cols, kept_col, kept_cnt and ws must be non-NULL");
  const TokWs w = tok_ws(dims, cfg, L.Sb, L.S, nnz);
  if (ws_bytes < w.total)
    return fail(DR_ERR_CAPACITY, "workspace of %zu bytes below the %zu required", ws_bytes, w.total);
  unsigned char* wsb = static_cast<unsigned char*>(ws);
  dr::TokParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.row_ptr = row_ptr;
  p.cols = cols;
  p.kept_col = kept_col;
  p.kept_cnt = kept_cnt;
  p.nnz = nnz;
  p.H = dims->heads;
  p.S = (int)L.S;
  p.Sb = L.Sb;
  p.Nf = cfg->num_frames;
  p.Nt = cfg->tokens_per_frame;
  p.Bs = cfg->block_size;
  p.L0 = dr::base_span(p.Nt);
  p.n_wg = w.n_wg;
  p.FR = w.FR;
  p.gamma = cfg->gamma;
  p.lambda = cfg->lambda;
  p.theta_c = cfg->theta_c;
  p.theta_m = cfg->theta_m;
  p.tau_near = tok->tau_near;
  p.tau_far = tok->tau_far;
  p.eps = tok->eps;
  p.scale = (float)(1.0 / (sqrt((double)dims->head_dim) * (double)tok->fused_heads));
  p.spin_limit = g_wait_limit.load(std::memory_order_relaxed);
  p.part = reinterpret_cast<dr::TokStat*>(wsb + w.part);
  p.thr = reinterpret_cast<float*>(wsb + w.thr);
  p.fmax = reinterpret_cast<unsigned long long*>(wsb + w.fmax);
  p.fn = reinterpret_cast<double*>(wsb + w.fn);
  p.served = reinterpret_cast<int*>(wsb + w.served);
  p.flags = wsb + w.flags;
  p.colsum = w.decide ? reinterpret_cast<float*>(wsb + w.colsum) : nullptr;
  p.und = w.decide ? wsb + w.und : nullptr;
  const hipError_t e = dr::launch_token_select(p, dims->batch, dims->head_dim, cfg->block_size, tok->fused_heads,
                                               stream);
  if (e != hipSuccess) return hip_fail(e, "token selection kernels");
  return ok();
}

namespace {

struct StaticWs {
  size_t state, hist, flags, total;
};

StaticWs static_ws(const dr_radial_cfg* c, long long nnz) {
  StaticWs w;
  const size_t nfp = (size_t)c->num_frames * c->num_frames;
  size_t off = 0;
  w.state = off;
  off = align256(off + nfp * sizeof(dr::StaticState));
  w.hist = off;
  off = align256(off + nfp * dr::kStaticBins * sizeof(uint32_t));
  w.flags = off;
  off = align256(off + (size_t)nnz);
  w.total = off;
  return w;
}

dr_status check_static(const dr_static_cfg* st, const dr_radial_cfg* c) {
  if (!st) return fail(DR_ERR_INVALID_ARG, "static config is NULL");
  if (!(st->rho_near >= 0.0 && st->rho_near <= 1.0) || !(st->rho_far >= 0.0 && st->rho_far <= 1.0))
    return fail(DR_ERR_INVALID_ARG, "rho_near and rho_far must lie in [0, 1]");
  if (c->tokens_per_frame < 32 || c->tokens_per_frame > 65535)
    return fail(DR_ERR_UNSUPPORTED, "static decay-state selection needs tokens_per_frame in [32, 65535]");
  if (c->num_frames > dr::kMaxTokenFrames)
    return fail(DR_ERR_UNSUPPORTED, "static decay-state selection supports num_frames <= %d", dr::kMaxTokenFrames);
  return DR_OK;
}

}  // namespace

dr_status dr_static_select_workspace(const dr_radial_cfg* cfg, int64_t nnz, size_t* bytes) {
  Layout L;
  dr_status st = check_radial(cfg, &L);
  if (st != DR_OK) return st;
  if (cfg->num_frames > dr::kMaxTokenFrames)
    return fail(DR_ERR_UNSUPPORTED, "static decay-state selection supports num_frames <= %d", dr::kMaxTokenFrames);
  if (nnz < 1 || nnz > (long long)L.Sb * L.Sb) return fail(DR_ERR_INVALID_ARG, "nnz %lld outside [1, S_b^2]", (long long)nnz);
  if (!bytes) return fail(DR_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = static_ws(cfg, nnz).total;
  return ok();
}

dr_status dr_static_select(const dr_dims* dims, const dr_radial_cfg* cfg, const dr_static_cfg* scfg,
                           const int32_t* row_ptr, const int32_t* cols, int64_t nnz, int32_t* kept_col,
                           int32_t* kept_cnt, void* ws, size_t ws_bytes, hipStream_t stream) {
  Layout L;
  dr_status st = check_radial(cfg, &L);
  if (st != DR_OK) return st;
  if ((st = check_dims(dims)) != DR_OK) return st;
  if ((st = check_static(scfg, cfg)) != DR_OK) return st;
  if ((st = check_nnz(nnz, L.Sb, dims)) != DR_OK) return st;
  if (!row_ptr || !cols || !kept_col || !kept_cnt || !ws)
    return fail(DR_ERR_INVALID_ARG, "row_ptr, cols, kept_col, kept_cnt and ws must be non-NULL");
  const StaticWs w = static_ws(cfg, nnz);
  if (ws_bytes < w.total)
    return fail(DR_ERR_CAPACITY, "workspace of %zu bytes below the %zu required", ws_bytes, w.total);
  unsigned char* wsb = static_cast<unsigned char*>(ws);
  dr::StaticParams p;
  p.row_ptr = row_ptr;
  p.cols = cols;
  p.nnz = nnz;
  p.S = (int)L.S;
  p.Sb = L.Sb;
  p.Nf = cfg->num_frames;
  p.Nt = cfg->tokens_per_frame;
  p.Bs = cfg->block_size;
  p.L0 = dr::base_span(p.Nt);
  p.gamma = cfg->gamma;
  p.lambda = cfg->lambda;
  p.theta_c = cfg->theta_c;
  p.theta_m = cfg->theta_m;
  p.rho_near = scfg->rho_near;
  p.rho_far = scfg->rho_far;
  p.seed_lo = (uint32_t)(scfg->seed & 0xffffffffu);
  p.seed_hi = (uint32_t)(scfg->seed >> 32);
  p.state = reinterpret_cast<dr::StaticState*>(wsb + w.state);
  p.hist = reinterpret_cast<uint32_t*>(wsb + w.hist);
  p.flags = wsb + w.flags;
  hipError_t e = dr::launch_static_select(p, stream);
  if (e != hipSuccess) return hip_fail(e, "static selection kernels");
  const dr::FlagCompact fc{row_ptr, cols, p.flags, 0, nnz, L.Sb, dims->heads, kept_col, kept_cnt};
  e = dr::launch_flag_compact(fc, dims->batch, stream);
  if (e != hipSuccess) return hip_fail(e, "kept-list compaction");
  return ok();
}

static dr_status proxy_impl(const void* o_ref, const void* o_test, int64_t n, const int32_t* kept_cnt, int64_t n_cnt,
                            bool with_loss, int64_t total_blocks, double alpha, double target, double* out, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  if (!o_ref || !o_test || !out || !ws) return fail(DR_ERR_INVALID_ARG, "o_ref, o_test, out and ws must be non-NULL");
  if (n < 1) return fail(DR_ERR_INVALID_ARG, "n must be >= 1");
  if (n_cnt < 0 || (n_cnt > 0 && !kept_cnt)) return fail(DR_ERR_INVALID_ARG, "n_cnt must be >= 0 (0 when kept_cnt is NULL)");
  if ((reinterpret_cast<uintptr_t>(o_ref) | reinterpret_cast<uintptr_t>(o_test)) & 15)
    return fail(DR_ERR_INVALID_ARG, "o_ref and o_test must be 16-byte aligned");
  static_assert(DR_PROXY_WS_BYTES == dr::kProxyPartials * 3 * sizeof(double), "proxy workspace size");
  if (ws_bytes < (size_t)DR_PROXY_WS_BYTES)
    return fail(DR_ERR_CAPACITY, "workspace of %zu bytes below the %d required", ws_bytes, DR_PROXY_WS_BYTES);
  dr::ProxyParams p;
  p.ref = static_cast<const uint16_t*>(o_ref);
  p.test = static_cast<const uint16_t*>(o_test);
  p.n = n;
  p.kept_cnt = kept_cnt;
  p.n_cnt = kept_cnt ? n_cnt : 0;
  p.partial = static_cast<double*>(ws);
  p.out = out;
  p.with_loss = with_loss ? 1 : 0;
  p.total_blocks = total_blocks;
  p.alpha = alpha;
  p.target = target;
  const hipError_t e = dr::launch_proxy_error(p, stream);
  if (e != hipSuccess) return hip_fail(e, "proxy error kernels");
  return ok();
}

dr_status dr_proxy_error(const void* o_ref, const void* o_test, int64_t n, const int32_t* kept_cnt, int64_t n_cnt,
                         double* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return proxy_impl(o_ref, o_test, n, kept_cnt, n_cnt, false, 0, 0.0, 0.0, out, ws, ws_bytes, stream);
}

dr_status dr_proxy_loss(const void* o_ref, const void* o_test, int64_t n, const int32_t* kept_cnt, int64_t n_cnt,
                        int64_t total_blocks, double alpha, double target, double* out, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  if (total_blocks < 1) return fail(DR_ERR_INVALID_ARG, "total_blocks must be >= 1");
  if (!isfinite(alpha) || alpha < 0.0) return fail(DR_ERR_INVALID_ARG, "alpha must be finite and >= 0");
  if (!isfinite(target)) return fail(DR_ERR_INVALID_ARG, "target must be finite");
  return proxy_impl(o_ref, o_test, n, kept_cnt, n_cnt, true, total_blocks, alpha, target, out, ws, ws_bytes, stream);
}

dr_status dr_set_wait_limit(int64_t polls) {
  if (polls < 0 || polls > (int64_t)0x7fffffff) return fail(DR_ERR_INVALID_ARG, "polls must be in [0, 2^31)");
  g_wait_limit.store(polls == 0 ? dr::kDefaultSpinLimit : (int)polls, std::memory_order_relaxed);
  return ok();
}

dr_status dr_wait_report(hipStream_t stream, uint32_t* flags) {
  if (!flags) return fail(DR_ERR_INVALID_ARG, "flags is NULL");
  unsigned a = 0, t = 0;
  hipError_t e = dr::take_wait_flags_attn(&a, stream);
  if (e != hipSuccess) return hip_fail(e, "reading the attention wait flags");
  e = dr::take_wait_flags_token(&t, stream);
  if (e != hipSuccess) return hip_fail(e, "reading the token-selection wait flags");
  *flags = a | t;
  if (*flags)
    return fail(DR_ERR_WAIT, "a bounded wait gave up (flags 0x%x): outputs of the ring kernels since the last report "
                             "are not valid", *flags);
  return ok();
}

static dr_status sparse_attn_impl(const dr_dims* dims, const dr_radial_cfg* cfg, const void* q, const void* k,
                                  const void* v, const int32_t* row_ptr, int64_t nnz, const int32_t* kept_col,
                                  const int32_t* kept_cnt, const int32_t* group_mode, float softmax_scale,
                                  void* out, hipStream_t stream) {
  Layout L;
  dr_status st = check_radial(cfg, &L);
  if (st != DR_OK) return st;
  if ((st = check_dims(dims)) != DR_OK) return st;
  if ((st = check_nnz(nnz, L.Sb, dims)) != DR_OK) return st;
  if (!row_ptr || !kept_col || !kept_cnt) return fail(DR_ERR_INVALID_ARG, "row_ptr, kept_col and kept_cnt must be non-NULL");
  dr::AttnParams p;
  if ((st = attn_common(dims, L.S, q, k, v, softmax_scale, out, &p)) != DR_OK) return st;
  p.row_ptr = row_ptr;
  p.kept_col = kept_col;
  p.kept_cnt = kept_cnt;
  p.group_mode = group_mode;
  p.grp = dr::make_qgroup(cfg->num_frames, cfg->tokens_per_frame, cfg->block_size, L.Sb);
  p.nnz = nnz;
  p.Sb = L.Sb;
  const hipError_t e = dr::launch_sparse_attn(p, dims->head_dim, cfg->block_size, stream);
  if (e != hipSuccess) return hip_fail(e, "sparse attention kernel");
  return ok();
}

dr_status dr_sparse_attn(const dr_dims* dims, const dr_radial_cfg* cfg, const void* q, const void* k,
                         const void* v, const int32_t* row_ptr, int64_t nnz, const int32_t* kept_col,
                         const int32_t* kept_cnt, float softmax_scale, void* out, hipStream_t stream) {
  return sparse_attn_impl(dims, cfg, q, k, v, row_ptr, nnz, kept_col, kept_cnt, nullptr, softmax_scale, out,
                          stream);
}

dr_status dr_sparse_attn_grouped(const dr_dims* dims, const dr_radial_cfg* cfg, const void* q, const void* k,
                                 const void* v, const int32_t* row_ptr, int64_t nnz, const int32_t* kept_col,
                                 const int32_t* kept_cnt, const int32_t* group_mode, float softmax_scale,
                                 void* out, hipStream_t stream) {
  if (!group_mode) return fail(DR_ERR_INVALID_ARG, "group_mode must be non-NULL");
  return sparse_attn_impl(dims, cfg, q, k, v, row_ptr, nnz, kept_col, kept_cnt, group_mode, softmax_scale, out,
                          stream);
}

int64_t dr_query_group_table(const dr_radial_cfg* cfg, int32_t mode, int32_t* table, int64_t cap) {
  Layout L;
  dr_status st = check_radial(cfg, &L);
  if (st != DR_OK) return -(int64_t)st;
  if (mode < 0 || mode >= dr::kGroupModes)
    return -(int64_t)fail(DR_ERR_INVALID_ARG, "mode %d outside [0, %d)", mode, dr::kGroupModes);
  const dr::QGroup g = dr::make_qgroup(cfg->num_frames, cfg->tokens_per_frame, cfg->block_size, L.Sb);
  const long long n = (long long)dr::group_count(g, mode) * g.QB;
  if (!table) {
    ok();
    return n;
  }
  if (cap < n)
    return -(int64_t)fail(DR_ERR_CAPACITY, "table of %lld entries below the %lld required", (long long)cap, n);
  for (int gi = 0; gi < dr::group_count(g, mode); ++gi)
    for (int s = 0; s < g.QB; ++s) table[(long long)gi * g.QB + s] = dr::group_block(g, mode, gi, s);
  ok();
  return n;
}

dr_status dr_query_groups_workspace(const dr_dims* dims, size_t* bytes) {
  dr_status st = check_dims(dims);
  if (st != DR_OK) return st;
  if (!bytes) return fail(DR_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = align256((size_t)dims->batch * dims->heads * dr::kGroupModes * sizeof(uint32_t));
  return ok();
}

static dr_status query_groups_impl(const dr_dims* dims, const dr_radial_cfg* cfg, const int32_t* row_ptr,
                                   int64_t nnz, const int32_t* kept_col, const int32_t* kept_cnt, int32_t* group_mode,
                                   void* ws, size_t ws_bytes, bool library_scratch, hipStream_t stream) {
  Layout L;
  dr_status st = check_radial(cfg, &L);
  if (st != DR_OK) return st;
  if ((st = check_dims(dims)) != DR_OK) return st;
  if ((st = check_nnz(nnz, L.Sb, dims)) != DR_OK) return st;
  if (!row_ptr || !kept_col || !kept_cnt || !group_mode)
    return fail(DR_ERR_INVALID_ARG, "row_ptr, kept_col, kept_cnt and group_mode must be non-NULL");
  if ((long long)dims->batch * dims->heads > 65535) return fail(DR_ERR_UNSUPPORTED, "batch * heads above 65535");
  if (library_scratch) {
    if ((long long)dims->batch * dims->heads > dr::kGroupScratchBH)
      return fail(DR_ERR_CAPACITY, "batch * heads = %lld above the %d the library's scratch holds",
                  (long long)dims->batch * dims->heads, dr::kGroupScratchBH);
    uint32_t* scratch = nullptr;
    const hipError_t e = dr::group_scratch(&scratch);
    if (e != hipSuccess) return hip_fail(e, "address of the grouping scratch on the current device");
    ws = scratch;
  } else {
    if (!ws) return fail(DR_ERR_INVALID_ARG, "ws must be non-NULL");
    const size_t need = align256((size_t)dims->batch * dims->heads * dr::kGroupModes * sizeof(uint32_t));
    if (ws_bytes < need)
      return fail(DR_ERR_CAPACITY, "workspace of %zu bytes below the %zu required", ws_bytes, need);
  }
  dr::GroupCostParams p;
  p.row_ptr = row_ptr;
  p.kept_col = kept_col;
  p.kept_cnt = kept_cnt;
  p.totals = static_cast<uint32_t*>(ws);
  p.group_mode = group_mode;
  p.grp = dr::make_qgroup(cfg->num_frames, cfg->tokens_per_frame, cfg->block_size, L.Sb);
  p.nnz = nnz;
  p.BH = dims->batch * dims->heads;
  p.gmax = 0;
  for (int m = 0; m < dr::kGroupModes; ++m) p.gmax = std::max(p.gmax, dr::group_count(p.grp, m));
  const hipError_t e = dr::launch_group_choice(p, stream);
  if (e != hipSuccess) return hip_fail(e, "query grouping kernels");
  return ok();
}

dr_status dr_query_groups(const dr_dims* dims, const dr_radial_cfg* cfg, const int32_t* row_ptr, int64_t nnz,
                          const int32_t* kept_col, const int32_t* kept_cnt, int32_t* group_mode, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  return query_groups_impl(dims, cfg, row_ptr, nnz, kept_col, kept_cnt, group_mode, ws, ws_bytes, false, stream);
}

dr_status dr_query_groups_noalloc(const dr_dims* dims, const dr_radial_cfg* cfg, const int32_t* row_ptr,
                                  int64_t nnz, const int32_t* kept_col, const int32_t* kept_cnt, int32_t* group_mode,
                                  hipStream_t stream) {
  return query_groups_impl(dims, cfg, row_ptr, nnz, kept_col, kept_cnt, group_mode, nullptr, 0, true, stream);
}

dr_status dr_attn(const dr_dims* dims, int32_t seq_len, const void* q, const void* k, const void* v,
                  float softmax_scale, void* out, hipStream_t stream) {
  dr_status st = check_dims(dims);
  if (st != DR_OK) return st;
  if (seq_len < 1) return fail(DR_ERR_INVALID_ARG, "seq_len must be >= 1");
  dr::AttnParams p;
  if ((st = attn_common(dims, seq_len, q, k, v, softmax_scale, out, &p)) != DR_OK) return st;
  p.row_ptr = nullptr;
  p.kept_col = nullptr;
  p.kept_cnt = nullptr;
  p.nnz = 0;
  p.Sb = (seq_len + 63) / 64;
  const hipError_t e = dr::launch_dense_attn(p, dims->head_dim, stream);
  if (e != hipSuccess) return hip_fail(e, "dense attention kernel");
  return ok();
}

const char* dr_status_string(dr_status s) {
  switch (s) {
    case DR_OK: return "ok";
    case DR_ERR_INVALID_ARG: return "invalid argument";
    case DR_ERR_UNSUPPORTED: return "unsupported configuration";
    case DR_ERR_CAPACITY: return "insufficient capacity";
    case DR_ERR_HIP: return "HIP error";
    case DR_ERR_WAIT: return "bounded wait gave up";
  }
  return "unknown status";
}

const char* dr_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
