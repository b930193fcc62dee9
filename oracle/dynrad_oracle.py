"""Plain CPU oracle for the DynamicRad block-sparse attention hot path.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or run this module. The product path (the HIP
library and its Python binding) never does, and this module imports nothing
from it.

It is written for a reader to check against the pages by eye: NumPy on the
host, float64 arithmetic throughout (inputs are bfloat16 values, exact in
float64), no blocking, fusion or reordering beyond what the definitions state.
Reference: "DynamicRad: Content-Adaptive Sparse Attention for Long Video
Diffusion" (arXiv 2604.20470), cited below as [DR] with section / equation.

Stages:

1. layout                 [DR] §3.1 "Notation"
2. distance_table         [DR] §3.1, Eqs. 1-5 (window width w(t), split stride sf(t))
3. candidate_row / candidate_csr
                          [DR] §3.1, Eqs. 6-7 and "Density control within blocks"
4. pool_blocks            block-importance estimate from mean-pooled Q and K
                          (the block-level form of [DR] §3.2 Eq. 9 / App. B Eq. 19)
5. block_scores           s(a, c) = mean-pooled Q_a . mean-pooled K_c / sqrt(D),
                          optionally averaged over the first H_f heads ([DR] Eq. 19)
6. select_static          static-ratio mode ([DR] §3.2), block form: keep the
                          top max(1, ceil(r * n)) candidates of a query block
7. select_dynamic         dynamic-threshold mode ([DR] §3.2), block form: keep
                          candidates in descending score order until their
                          cumulative softmax mass reaches tau; at least one kept
                          ([DR] §3.2 safeguard (ii), App. B fallback)
8. sparse_attention       [DR] §3.3 Eqs. 12-13 with the block mask broadcast to
                          tokens and eps -> 0 (masked keys get exactly zero weight)
9. masked_attention_dense the same Eq. 13 written over a full token mask (tiny
                          shapes), and dense_attention (no mask, [DR] App. A Eq. 16)

Readings where the pages leave a step open are stated at each function.
"""

from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

EPS_SPLIT = 1e-6      # the epsilon of Eq. 5 (value not given on the pages)
COUNT_GUARD = 1e-9    # guard in ceil(r * n - guard) against representation error

__all__ = [
    "layout", "distance_table", "token_frame_and_index", "candidate_row", "candidate_csr",
    "pool_blocks", "block_scores", "select_static", "select_dynamic", "select_row",
    "selection_margin", "select_all", "sparse_attention", "sparse_attention_rows",
    "dense_attention", "masked_attention_dense", "kept_to_block_mask",
]


# ---------------------------------------------------------------------------
# 1. Layout ([DR] §3.1 Notation): S = N_f * N_t tokens, padded to
#    S' = ceil(S / B_s) * B_s; S_b = S' / B_s blocks.
# ---------------------------------------------------------------------------
def layout(num_frames: int, tokens_per_frame: int, block_size: int) -> dict:
    S = num_frames * tokens_per_frame
    S_b = -(-S // block_size)
    return {"S": S, "S_pad": S_b * block_size, "S_b": S_b}


def token_frame_and_index(s, tokens_per_frame: int):
    """Token s sits in frame floor(s / N_t) at local spatial index s mod N_t
    (frames are stored one after another; Eq. 7 uses the 1-D local index)."""
    s = np.asarray(s, dtype=np.int64)
    return s // tokens_per_frame, s % tokens_per_frame


# ---------------------------------------------------------------------------
# 2. Per-distance table ([DR] §3.1, Eqs. 1-5).
# ---------------------------------------------------------------------------
def _group_index(t: int) -> int:
    """Eq. 1: B(t) = floor(log2 t) + 1 for t >= 1, which is the number of
    binary digits of t (exact for every integer, unlike a float log2)."""
    return int(t).bit_length()


def _base_span(tokens_per_frame: int) -> int:
    """Eq. 1: L0 = 2^ceil(log2 N_t), the next power of two >= N_t."""
    L0 = 1
    while L0 < tokens_per_frame:
        L0 *= 2
    return L0


def distance_table(num_frames: int, tokens_per_frame: int, block_size: int,
                   gamma: float, lam: float, eps: float = EPS_SPLIT) -> Tuple[np.ndarray, np.ndarray]:
    """Window width w(t) and split stride sf(t) for temporal distances t < N_f.

    * t = 0 (same frame): dense ([DR] §3.1 after Eq. 1; §3.2; Algorithm 1
      marks the diagonal): w = N_t, sf = 1.
    * t >= 1: L(t) = L0 / 2^B(t) * gamma (Eq. 2);
      w = N_t if t <= 1 else max(B_s, round(L(t))) (Eq. 3);
      L_split(t) = L0 / 2^B(t) * lambda (Eq. 4);
      sf(t) = max(1, floor(B_s / (L_split(t) + eps))) (Eq. 5).

    Readings: round(x) in Eq. 3 is floor(x + 1/2) (ties up); eps = 1e-6; all in
    float64 with the operation order written here. Eq. 5 is applied at every
    t >= 1, including t = 1, as Algorithm 1 does; only t = 0 is exempt.
    """
    L0 = _base_span(tokens_per_frame)
    w = np.zeros(num_frames, dtype=np.int64)
    sf = np.ones(num_frames, dtype=np.int64)
    for t in range(num_frames):
        if t == 0:
            w[t] = tokens_per_frame
            sf[t] = 1
            continue
        B = _group_index(t)
        span = float(L0) / float(2 ** B)
        decay = span * gamma                       # Eq. 2
        if t <= 1:
            w[t] = tokens_per_frame                # Eq. 3, intra & adjacent
        else:
            w[t] = max(block_size, int(math.floor(decay + 0.5)))   # Eq. 3
        split = span * lam                         # Eq. 4
        sf[t] = max(1, int(math.floor(block_size / (split + eps))))  # Eq. 5
    return w, sf


# ---------------------------------------------------------------------------
# 3. Candidate blocks ([DR] §3.1 Eqs. 6-7 and "Density control within blocks").
#    Token pair (q, k) is a candidate iff its frame pair is retained
#    (t mod sf(t) = 0, Eq. 6) and |u_q - u_k| <= w(t) (Eq. 7).
#    Block pair (a, b), a = query block, b = key block: a key token (column) of
#    b is active iff (number of query tokens of a paired with it) / (number of
#    query tokens of a) exceeds theta_c; the block is a candidate iff (active
#    columns) / (key tokens of b) exceeds theta_m. Padding tokens (s >= S) are
#    not tokens: they count in neither numerator nor denominator.
# ---------------------------------------------------------------------------
def candidate_row(a: int, num_frames: int, tokens_per_frame: int, block_size: int,
                  gamma: float, lam: float, theta_c: float = 0.0, theta_m: float = 0.0,
                  table=None) -> np.ndarray:
    """Ascending key-block indices b that are candidates for query block a."""
    lay = layout(num_frames, tokens_per_frame, block_size)
    S, S_b = lay["S"], lay["S_b"]
    w, sf = table if table is not None else distance_table(
        num_frames, tokens_per_frame, block_size, gamma, lam)
    q = np.arange(a * block_size, min((a + 1) * block_size, S))
    k = np.arange(S)
    fq, uq = token_frame_and_index(q, tokens_per_frame)
    fk, uk = token_frame_and_index(k, tokens_per_frame)
    t = np.abs(fq[:, None] - fk[None, :])                       # temporal distance
    retained = (t % sf[t]) == 0                                 # Eq. 6
    within = np.abs(uq[:, None] - uk[None, :]) <= w[t]          # Eq. 7
    pair = retained & within
    count = pair.sum(axis=0)                                     # per key token
    col_ratio = count.astype(np.float64) / float(len(q))
    active = col_ratio > theta_c
    pad = S_b * block_size - S
    active_blocks = np.concatenate([active, np.zeros(pad, dtype=bool)]).reshape(S_b, block_size)
    n_valid = np.full(S_b, block_size, dtype=np.int64)
    n_valid[-1] = S - (S_b - 1) * block_size
    frac = active_blocks.sum(axis=1).astype(np.float64) / n_valid.astype(np.float64)
    return np.nonzero(frac > theta_m)[0].astype(np.int64)


def candidate_csr(num_frames: int, tokens_per_frame: int, block_size: int, gamma: float,
                  lam: float, theta_c: float = 0.0, theta_m: float = 0.0):
    """Candidate set of every query block as CSR: (row_ptr[S_b + 1], cols[nnz])."""
    S_b = layout(num_frames, tokens_per_frame, block_size)["S_b"]
    table = distance_table(num_frames, tokens_per_frame, block_size, gamma, lam)
    rows = [candidate_row(a, num_frames, tokens_per_frame, block_size, gamma, lam,
                          theta_c, theta_m, table=table) for a in range(S_b)]
    row_ptr = np.zeros(S_b + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    cols = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)
    return row_ptr, cols


# ---------------------------------------------------------------------------
# 4-5. Block-importance estimate: mean-pooled Q and K per block, then
#      s(a, c) = Qbar_a . Kbar_c / sqrt(D) on the candidates. This is the
#      block-level form of the proxy logits of [DR] §3.2 Eq. 9 (1/sqrt(d_k)
#      scaling); with fused heads, the mean over the first H_f heads
#      ([DR] Eq. 19, App. B "Head Fusion Proxy") and one mask for all heads.
# ---------------------------------------------------------------------------
def pool_blocks(x: np.ndarray, block_size: int) -> np.ndarray:
    """x: [S, D] -> [S_b, D] float64: mean of each block's valid (non-padding) rows."""
    x = np.asarray(x, dtype=np.float64)
    S = x.shape[0]
    S_b = -(-S // block_size)
    out = np.empty((S_b, x.shape[1]), dtype=np.float64)
    for a in range(S_b):
        out[a] = x[a * block_size:min((a + 1) * block_size, S)].mean(axis=0)
    return out


def block_scores(qbar: np.ndarray, kbar: np.ndarray, row_ptr, cols) -> np.ndarray:
    """Scores of the candidate entries, in CSR order. qbar, kbar: [S_b, D]."""
    D = qbar.shape[1]
    out = np.empty(len(cols), dtype=np.float64)
    for a in range(len(row_ptr) - 1):
        c = cols[row_ptr[a]:row_ptr[a + 1]]
        out[row_ptr[a]:row_ptr[a + 1]] = (kbar[c] @ qbar[a]) / math.sqrt(D)
    return out


def fused_scores(qbars: Sequence[np.ndarray], kbars: Sequence[np.ndarray], row_ptr, cols) -> np.ndarray:
    """[DR] Eq. 19: average of the per-head scores over the given heads."""
    s = [block_scores(qb, kb, row_ptr, cols) for qb, kb in zip(qbars, kbars)]
    return np.mean(np.stack(s), axis=0)


# ---------------------------------------------------------------------------
# 6-7. Dual-mode selection within one query block's candidate row.
#      Order: score descending, ties to the lower key-block index.
# ---------------------------------------------------------------------------
def _descending_order(scores: np.ndarray, cols: np.ndarray) -> np.ndarray:
    return np.lexsort((cols, -scores))


def static_count(n: int, ratio: float) -> int:
    """k = max(1, ceil(r * n)), evaluated as ceil(r * n - 1e-9) in float64 so
    that representation error in r cannot add a block (the paper's static mode
    keeps max(1, floor(|P| * rho)) sampled pairs; the block form keeps the
    top ceil(r * n) candidates)."""
    return max(1, int(math.ceil(ratio * n - COUNT_GUARD)))


def select_static(scores: np.ndarray, cols: np.ndarray, ratio: float) -> np.ndarray:
    """Static-ratio mode: keep the k highest-scoring candidates; ascending output."""
    n = len(cols)
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    order = _descending_order(scores, cols)
    return np.sort(cols[order[:static_count(n, ratio)]])


def _softmax(scores: np.ndarray) -> np.ndarray:
    e = np.exp(scores - scores.max())
    return e / e.sum()


def dynamic_count(scores: np.ndarray, cols: np.ndarray, tau: float) -> int:
    """Smallest k such that the k top-scoring candidates hold softmax mass >= tau
    (softmax over the row's candidates, raw logits); k = n when tau >= 1."""
    n = len(cols)
    if tau >= 1.0:
        return n
    order = _descending_order(scores, cols)
    cum = np.cumsum(_softmax(scores)[order])
    hit = np.nonzero(cum >= tau)[0]
    return int(hit[0]) + 1 if len(hit) else n


def select_dynamic(scores: np.ndarray, cols: np.ndarray, tau: float) -> np.ndarray:
    """Dynamic-threshold mode: keep candidates in descending score order until
    their cumulative softmax mass reaches tau (at least one is always kept)."""
    n = len(cols)
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    order = _descending_order(scores, cols)
    return np.sort(cols[order[:dynamic_count(scores, cols, tau)]])


def select_row(scores, cols, mode: str, ratio: float = 1.0, tau: float = 1.0) -> np.ndarray:
    if mode == "static":
        return select_static(scores, cols, ratio)
    if mode == "dynamic":
        return select_dynamic(scores, cols, tau)
    raise ValueError(mode)


def selection_margin(scores: np.ndarray, cols: np.ndarray, mode: str, ratio: float = 1.0,
                     tau: float = 1.0) -> float:
    """How far the row's decision is from flipping.

    Sorted scores s_1 >= s_2 >= ..., k kept. Static: s_k - s_{k+1} (inf if
    k = n). Dynamic: min(s_k - s_{k+1}, cum_k - tau, tau - cum_{k-1}) with
    cum_0 = 0 (inf if tau >= 1).
    """
    n = len(cols)
    if n == 0:
        return math.inf
    order = _descending_order(scores, cols)
    s = scores[order]
    if mode == "static":
        k = static_count(n, ratio)
        return math.inf if k >= n else float(s[k - 1] - s[k])
    if tau >= 1.0:
        return math.inf
    cum = np.cumsum(_softmax(scores)[order])
    k = dynamic_count(scores, cols, tau)
    m = float(cum[k - 1] - tau)
    m = min(m, float(tau - (cum[k - 2] if k >= 2 else 0.0)))
    if k < n:
        m = min(m, float(s[k - 1] - s[k]))
    return m


def select_all(scores: np.ndarray, row_ptr, cols, mode: str, ratio: float = 1.0,
               tau: float = 1.0) -> Tuple[List[np.ndarray], np.ndarray]:
    """Kept lists of every row plus each row's margin."""
    kept, margins = [], np.empty(len(row_ptr) - 1)
    for a in range(len(row_ptr) - 1):
        lo, hi = row_ptr[a], row_ptr[a + 1]
        kept.append(select_row(scores[lo:hi], cols[lo:hi], mode, ratio, tau))
        margins[a] = selection_margin(scores[lo:hi], cols[lo:hi], mode, ratio, tau)
    return kept, margins


# ---------------------------------------------------------------------------
# 8-9. Attention ([DR] §3.3 Eqs. 12-13). A = Q K^T / sqrt(d_k) (or the given
#      scale); the block mask is broadcast to tokens and applied as
#      log(M + eps) with eps -> 0, i.e. masked keys get weight exactly 0.
#      Padding keys are never attended; padding queries produce no output.
# ---------------------------------------------------------------------------
def _softmax_rows(logits: np.ndarray) -> np.ndarray:
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=1, keepdims=True)


def sparse_attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, block_size: int,
                          kept: Sequence[np.ndarray], query_blocks: Sequence[int],
                          scale: float = None) -> np.ndarray:
    """Outputs of the valid tokens of the given query blocks, stacked in order."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    S, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    outs = []
    for a in query_blocks:
        rows = np.arange(a * block_size, min((a + 1) * block_size, S))
        keys = np.concatenate([np.arange(b * block_size, min((b + 1) * block_size, S))
                               for b in kept[a]])
        p = _softmax_rows((q[rows] @ k[keys].T) * scale)
        outs.append(p @ v[keys])
    return np.concatenate(outs) if outs else np.zeros((0, D))


def sparse_attention(q, k, v, block_size: int, kept: Sequence[np.ndarray], scale: float = None) -> np.ndarray:
    """[S, D] output of block-sparse attention with per-query-block kept lists."""
    return sparse_attention_rows(q, k, v, block_size, kept, range(len(kept)), scale)


def dense_attention(q, k, v, scale: float = None, rows=None) -> np.ndarray:
    """Softmax(Q K^T * scale) V over all keys ([DR] App. A, the dense baseline)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    scale = 1.0 / math.sqrt(q.shape[1]) if scale is None else scale
    qr = q if rows is None else q[rows]
    return _softmax_rows((qr @ k.T) * scale) @ v


def kept_to_block_mask(kept: Sequence[np.ndarray], S_b: int) -> np.ndarray:
    M = np.zeros((S_b, S_b), dtype=bool)
    for a, ks in enumerate(kept):
        M[a, np.asarray(ks, dtype=np.int64)] = True
    return M


def masked_attention_dense(q, k, v, block_size: int, block_mask: np.ndarray, scale: float = None) -> np.ndarray:
    """Eq. 13 written literally on a full S' x S' token mask (tiny shapes only):
    Softmax(A + log(M~)) V with log 0 = -inf; padding rows/columns are dropped."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    S, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    S_b = block_mask.shape[0]
    tok = np.kron(block_mask.astype(np.float64), np.ones((block_size, block_size)))[:S, :S]
    A = (q @ k.T) * scale
    with np.errstate(divide="ignore"):
        A = A + np.log(tok)
    return _softmax_rows(A) @ v
