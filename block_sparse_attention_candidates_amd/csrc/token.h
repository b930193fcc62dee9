// Token-level dynamic-threshold selection ([DR] §3.2 Eqs. 9-11): parameters
// and launch shared by token_select.hip and the C ABI. [DR] = "DynamicRad:
// Content-Adaptive Sparse Attention for Long Video Diffusion", arXiv 2604.20470.
#pragma once
#include "dr_internal.h"

namespace dr {

constexpr int kTokSplit = 4;         // workgroups sharing one query group's walk of key blocks

// Statistics of a set of scores: count, mean, sum of squared deviations, and
// the highest score packed with its position ((order key << 32) | ~position).
struct TokStat {
  double n, mean, m2;
  unsigned long long mx;
};

struct TokParams {
  const uint16_t* q;
  const uint16_t* k;
  const int32_t* row_ptr;
  const int32_t* cols;
  int32_t* kept_col;
  int32_t* kept_cnt;
  long long nnz;
  int H, S, Sb, Nf, Nt, Bs, L0;
  int n_wg;            // workgroups per batch element (256 query tokens each)
  int FR;              // query frames a workgroup can span
  double gamma, lambda, theta_c, theta_m, tau_near, tau_far, eps;
  float scale;         // 1 / (sqrt(d_k) * H_f)
  int spin_limit;      // polls before a bounded wait gives up (>= 1)
  int nb;              // key-block ring buffers (set at launch)
  // workspace
  TokStat* part;       // [B][n_wg][kTokSplit][FR][Nf] workgroup partials
  float* thr;          // [B][Nf][Nf] threshold in score units (+inf: no t > 1 pair)
  unsigned long long* fmax;  // [B][Nf][Nf] highest score and position
  double* fn;          // [B][Nf][Nf] size of P(i, j) for t > 1 (0: none)
  int* served;         // [B][Nf][Nf] 1 if some t > 1 pair is selected
  unsigned char* flags;  // [B][nnz] block decision per candidate entry
  // B_s <= 64 only (else null): per candidate entry and 32 x 32 tile of it
  // whose query rows lie in one frame, each key column's sum of logits in P
  // and of their squares (float32, [B][nnz][(B_s/32)^2][32][2]); and whether
  // the mark pass must decide the entry ([B][nnz], 1) or its flag is fixed (0)
  float* colsum;
  unsigned char* und;
};

size_t token_lds_bytes(int D, int Bs, int Hf, int Sb, int Nf, int FR);

hipError_t launch_token_select(const TokParams& p, int B, int D, int Bs, int Hf, hipStream_t stream);

}  // namespace dr
