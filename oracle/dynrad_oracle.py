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
10. token_selection / token_select
                          the paper's token-level dynamic-threshold mode ([DR] §3.2
                          Eqs. 9-11 with safeguard (ii), Algorithm 1): fused-head
                          logits per candidate token pair, z-normalised per frame
                          pair, decay-state thresholds, top-pair fallback, then the
                          same (theta_c, theta_m) aggregation to blocks as step 3
11. static_select         the paper's decay-state static-ratio mode ([DR] §3.2
                          Eq. 8, Algorithm 1): per retained frame pair a uniform
                          sample of max(1, floor(|P(i, j)| * rho)) candidate pairs
                          drawn with a seeded counter-based generator
                          (Philox4x32-10), then the same aggregation to blocks
12. proxy_*               the proxy-task objective ([DR] App. C.2 / C.4, Eq. 22):
                          normalised squared error of the sparse attention
                          matrix against the dense one plus a sparsity penalty;
                          exactly on tiny inputs, and through a random probe
                          (the form the attention kernels can evaluate)

Readings where the pages leave a step open are stated at each function.
"""

from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

EPS_SPLIT = 1e-6      # the epsilon of Eq. 5 (value not given on the pages)
EPS_NORM = 1e-6       # the epsilon of Eq. 10 (value not given on the pages)
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


# ---------------------------------------------------------------------------
# 10. Token-level dynamic-threshold selection ([DR] §3.2 "Dynamic-threshold
#     mode", Eqs. 9-11, "Global thresholding with safeguards"; Algorithm 1).
#     Small shapes only: every token pair's score is materialised.
# ---------------------------------------------------------------------------
def decay_length(t: int, tokens_per_frame: int, gamma: float) -> float:
    """Eq. 2: L(t) = L0 / 2^B(t) * gamma, for t >= 1 (same operation order as
    distance_table)."""
    return float(_base_span(tokens_per_frame)) / float(2 ** _group_index(t)) * gamma


def _fused(x_heads):
    return [np.asarray(x, dtype=np.float64) for x in x_heads]


def token_scores_block(q_heads, k_heads, rows: slice, cols: slice, scale: float) -> np.ndarray:
    """Eq. 9 on a sub-matrix: s(u, v) = (1 / H_f) sum_h Q_u^(h) . K_v^(h) * scale
    for query tokens `rows` and key tokens `cols` (scale = 1 / sqrt(d_k))."""
    acc = None
    for qh, kh in zip(q_heads, k_heads):
        part = (qh[rows] @ kh[cols].T) * scale
        acc = part if acc is None else acc + part
    return acc / float(len(q_heads))


def token_frame_stats(q_heads, k_heads, num_frames: int, tokens_per_frame: int, block_size: int,
                      gamma: float, lam: float, tau_near: float, tau_far: float,
                      eps: float = EPS_NORM, scale: float = None, top2: dict = None,
                      query_frames=None) -> dict:
    """Per frame pair (i, j) with t = |i - j| > 1 that is retained (Eq. 6):
    (mu, sigma, tau, fallback) where mu and sigma are the mean and standard
    deviation of s over P(i, j) (Eqs. 7, 9, 10), tau = tau_near if L(t) >= B_s
    else tau_far (Eq. 11), and fallback = (u, v) of the highest-scoring pair if
    no pair reaches tau, else None (safeguard (ii)).
    Readings: sigma is the population standard deviation (divide by |P|);
    eps = 1e-6; a tie for the highest score goes to the first pair in (u, v)
    order. If top2 is a dict, it receives the two highest scores of each
    frame pair (for token_select_decisive). query_frames, if given, limits
    the result to frame pairs (i, j) with i in it (each pair's statistics
    depend on that pair alone)."""
    q_heads, k_heads = _fused(q_heads), _fused(k_heads)
    scale = 1.0 / math.sqrt(q_heads[0].shape[1]) if scale is None else scale
    w, sf = distance_table(num_frames, tokens_per_frame, block_size, gamma, lam)
    Nt = tokens_per_frame
    u = np.arange(Nt)
    stats = {}
    for i in (range(num_frames) if query_frames is None else sorted(query_frames)):
        for j in range(num_frames):
            t = abs(i - j)
            if t <= 1 or t % sf[t] != 0:
                continue
            P = np.abs(u[:, None] - u[None, :]) <= w[t]
            sv = token_scores_block(q_heads, k_heads, slice(i * Nt, (i + 1) * Nt), slice(j * Nt, (j + 1) * Nt), scale)
            vals = sv[P]
            mu = vals.mean()
            sigma = math.sqrt(((vals - mu) ** 2).mean())
            tau = tau_near if decay_length(t, Nt, gamma) >= block_size else tau_far
            z = (sv - mu) / (sigma + eps)
            fallback = None
            if not (P & (z >= tau)).any():
                masked = np.where(P, sv, -np.inf)
                fallback = tuple(int(x) for x in np.unravel_index(int(np.argmax(masked)), masked.shape))
            stats[(i, j)] = (mu, sigma, tau, fallback)
            if top2 is not None:
                srt = np.partition(vals, len(vals) - 2)[-2:] if len(vals) > 1 else np.array([-np.inf, vals[0]])
                top2[(i, j)] = (float(srt.max()), float(srt.min()))
    return stats


def token_selected_rows(q_heads, k_heads, rows: slice, num_frames: int, tokens_per_frame: int,
                        block_size: int, gamma: float, lam: float, stats: dict,
                        eps: float = EPS_NORM, scale: float = None) -> np.ndarray:
    """Selected token pairs [len(rows), S] for the query tokens `rows`
    (Algorithm 1): for each frame pair, t mod sf(t) != 0 -> none (Eq. 6);
    t <= 1 -> all of P(i, j) (tau = -inf, Eq. 11; t = 0 is dense attention);
    otherwise the pairs of P(i, j) with (s - mu) / (sigma + eps) >= tau, or,
    if no pair of the frame pair reaches tau, its highest-scoring pair."""
    q_heads, k_heads = _fused(q_heads), _fused(k_heads)
    scale = 1.0 / math.sqrt(q_heads[0].shape[1]) if scale is None else scale
    w, sf = distance_table(num_frames, tokens_per_frame, block_size, gamma, lam)
    Nt = tokens_per_frame
    S = num_frames * Nt
    sel = np.zeros((rows.stop - rows.start, S), dtype=bool)
    qtok = np.arange(rows.start, rows.stop)
    fq, uq = token_frame_and_index(qtok, Nt)
    ukey = np.arange(Nt)
    for i in np.unique(fq):
        r = np.nonzero(fq == i)[0]
        for j in range(num_frames):
            t = abs(int(i) - j)
            if t % sf[t] != 0:
                continue
            P = np.abs(uq[r][:, None] - ukey[None, :]) <= w[t]
            cols = slice(j * Nt, (j + 1) * Nt)
            if t <= 1:
                sel[r, cols] = P
                continue
            mu, sigma, tau, fallback = stats[(int(i), j)]
            if fallback is None:
                sv = token_scores_block(q_heads, k_heads, slice(rows.start + r[0], rows.start + r[-1] + 1), cols, scale)
                sel[r, cols] = P & ((sv - mu) / (sigma + eps) >= tau)
            else:
                fu, fv = fallback
                hit = np.nonzero(uq[r] == fu)[0]
                if len(hit):
                    sel[r[hit[0]], j * Nt + fv] = True
    return sel


def aggregate_block_rows(sel_rows: np.ndarray, row_start: int, block_size: int, S: int,
                         theta_c: float = 0.0, theta_m: float = 0.0) -> List[np.ndarray]:
    """Kept key blocks of the query blocks covered by sel_rows (which starts at
    the first token of a block) under the density control of [DR] §3.1 (the
    rule of step 3): a key token of block b is active for query block a iff the
    fraction of a's valid query tokens paired with it exceeds theta_c; the block
    pair is kept iff the fraction of b's valid key tokens that are active exceeds
    theta_m. Reading: the selected pairs of all frame pairs a block pair spans
    are merged first (Algorithm 1 merges into M_b)."""
    S_b = -(-S // block_size)
    out = []
    n_rows = sel_rows.shape[0]
    for r0 in range(0, n_rows, block_size):
        blk = sel_rows[r0:min(r0 + block_size, n_rows)]
        nq = blk.shape[0]
        cnt = blk.sum(axis=0)
        active = (cnt.astype(np.float64) / float(nq)) > theta_c
        kept = []
        for b in range(S_b):
            lo, hi = b * block_size, min((b + 1) * block_size, S)
            if (active[lo:hi].sum() / float(hi - lo)) > theta_m:
                kept.append(b)
        out.append(np.asarray(kept, dtype=np.int64))
    return out


def token_select_rows(q_heads, k_heads, blocks, num_frames: int, tokens_per_frame: int, block_size: int,
                      gamma: float, lam: float, tau_near: float, tau_far: float, theta_c: float = 0.0,
                      theta_m: float = 0.0, eps: float = EPS_NORM, scale: float = None, stats: dict = None):
    """Kept key blocks (ascending) of the given query blocks under the
    token-level dynamic-threshold mode; one mask serves every head."""
    S = num_frames * tokens_per_frame
    if stats is None:
        stats = token_frame_stats(q_heads, k_heads, num_frames, tokens_per_frame, block_size, gamma, lam,
                                  tau_near, tau_far, eps, scale)
    out = []
    for a in blocks:
        rows = slice(a * block_size, min((a + 1) * block_size, S))
        sel = token_selected_rows(q_heads, k_heads, rows, num_frames, tokens_per_frame, block_size, gamma, lam,
                                  stats, eps, scale)
        out.append(aggregate_block_rows(sel, rows.start, block_size, S, theta_c, theta_m)[0])
    return out


def token_select(q_heads, k_heads, num_frames: int, tokens_per_frame: int, block_size: int,
                 gamma: float, lam: float, tau_near: float, tau_far: float, theta_c: float = 0.0,
                 theta_m: float = 0.0, eps: float = EPS_NORM, scale: float = None) -> List[np.ndarray]:
    """Kept key blocks of every query block (ascending)."""
    S_b = -(-(num_frames * tokens_per_frame) // block_size)
    return token_select_rows(q_heads, k_heads, range(S_b), num_frames, tokens_per_frame, block_size, gamma, lam,
                             tau_near, tau_far, theta_c, theta_m, eps, scale)


def token_select_decisive(q_heads, k_heads, blocks, num_frames: int, tokens_per_frame: int, block_size: int,
                          gamma: float, lam: float, tau_near: float, tau_far: float, margin: float,
                          eps: float = EPS_NORM, scale: float = None, stats: dict = None,
                          top2: dict = None) -> List[np.ndarray]:
    """For each given query block, a bool per key block: True where no
    token-level decision of the block pair can flip when every z moves by less
    than `margin` and every score by less than `margin` * (sigma + eps) / 2
    (two scores then keep their order unless they are within `margin` *
    (sigma + eps) of each other). Unsure are pairs of P (t > 1) within `margin`
    of their threshold, and every pair of a frame pair whose fallback is in
    doubt (its highest z within `margin` of tau, or no pair passing and a
    runner-up score within `margin` * (sigma + eps) of the highest). Pinned by
    hand-worked cases and by brute-force perturbation of tiny layouts."""
    q_heads, k_heads = _fused(q_heads), _fused(k_heads)
    scale = 1.0 / math.sqrt(q_heads[0].shape[1]) if scale is None else scale
    if stats is None:
        stats = token_frame_stats(q_heads, k_heads, num_frames, tokens_per_frame, block_size, gamma, lam,
                                  tau_near, tau_far, eps, scale)
    w, sf = distance_table(num_frames, tokens_per_frame, block_size, gamma, lam)
    Nt = tokens_per_frame
    S = num_frames * Nt
    S_b = -(-S // block_size)
    ukey = np.arange(Nt)
    doubtful = {}
    for (i, j), (mu, sigma, tau, fb) in stats.items():
        if top2 is not None:
            t1, t2 = top2[(i, j)]
        else:
            t = abs(i - j)
            P = np.abs(ukey[:, None] - ukey[None, :]) <= w[t]
            sv = token_scores_block(q_heads, k_heads, slice(i * Nt, (i + 1) * Nt), slice(j * Nt, (j + 1) * Nt),
                                    scale)
            top = np.sort(sv[P])[::-1]
            t1, t2 = top[0], (top[1] if len(top) > 1 else -np.inf)
        zmax = (t1 - mu) / (sigma + eps)
        doubtful[(i, j)] = abs(zmax - tau) <= margin or (zmax < tau and t1 - t2 <= margin * (sigma + eps))
    out = []
    for a in blocks:
        rows = slice(a * block_size, min((a + 1) * block_size, S))
        qtok = np.arange(rows.start, rows.stop)
        fq, uq = token_frame_and_index(qtok, Nt)
        unsure = np.zeros((len(qtok), S), dtype=bool)
        for i in np.unique(fq):
            r = np.nonzero(fq == i)[0]
            for j in range(num_frames):
                st = stats.get((int(i), j))
                if st is None:
                    continue
                mu, sigma, tau, fb = st
                t = abs(int(i) - j)
                P = np.abs(uq[r][:, None] - ukey[None, :]) <= w[t]
                cols = slice(j * Nt, (j + 1) * Nt)
                if doubtful[(int(i), j)]:
                    unsure[r, cols] = P
                    continue
                sv = token_scores_block(q_heads, k_heads, slice(rows.start + r[0], rows.start + r[-1] + 1), cols, scale)
                unsure[r, cols] = P & (np.abs((sv - mu) / (sigma + eps) - tau) <= margin)
        dec = np.ones(S_b, dtype=bool)
        for b in range(S_b):
            dec[b] = not unsure[:, b * block_size:min((b + 1) * block_size, S)].any()
        out.append(dec)
    return out


# ---------------------------------------------------------------------------
# 11. Decay-state static-ratio selection ([DR] §3.2 "Static-ratio mode", Eq. 8,
#     Algorithm 1). For each retained frame pair (i, j) (t mod sf(t) = 0):
#     t <= 1 keeps all of P(i, j) (rho = 1; t = 0 is dense attention);
#     t > 1 keeps k = max(1, floor(|P(i, j)| * rho)) pairs of P(i, j) drawn
#     uniformly, rho = rho_1 if L(t) >= B_s (near) else rho_2 (far). The
#     selected pairs are aggregated to blocks as in steps 3 and 10.
#
#     Reading of the uniform sampling under a fixed seed (the pages
#     name no generator): pair (u, v) of P(i, j) gets the 32-bit word number
#     (v mod 4) of Philox4x32-10 applied to the counter (u, floor(v / 4), i, j)
#     under the key (seed mod 2^32, seed div 2^32); the k pairs with the
#     smallest (word, u * N_t + v) are kept. The k smallest of independent
#     uniform keys form a uniformly random k-subset.
#     Reading of floor(|P| * rho): evaluated in float64 with the same 1e-9
#     guard as the block form's count (floor(|P| * rho + 1e-9)).
# ---------------------------------------------------------------------------
PHILOX_M = (0xD2511F53, 0xCD9E8D57)   # round multipliers
PHILOX_W = (0x9E3779B9, 0xBB67AE85)   # key schedule increments
_U32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel
    Random Numbers: As Easy as 1, 2, 3", SC 2011), elementwise over arrays of
    32-bit counters. One round: the products M0 * c0 and M1 * c2 (64-bit) give
    the new counter (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
    lo(M0 c0)); the key advances by (W0, W1) before every round after the first.
    Returns the four output words as uint64 arrays holding 32-bit values."""
    c = [np.asarray(x, dtype=np.uint64) & _U32 for x in (c0, c1, c2, c3)]
    k = [int(k0) & 0xFFFFFFFF, int(k1) & 0xFFFFFFFF]
    for r in range(10):
        if r:
            k = [(k[0] + PHILOX_W[0]) & 0xFFFFFFFF, (k[1] + PHILOX_W[1]) & 0xFFFFFFFF]
        p0 = np.uint64(PHILOX_M[0]) * c[0]
        p1 = np.uint64(PHILOX_M[1]) * c[2]
        c = [(p1 >> np.uint64(32)) ^ c[1] ^ np.uint64(k[0]), p1 & _U32,
             (p0 >> np.uint64(32)) ^ c[3] ^ np.uint64(k[1]), p0 & _U32]
    return c


def static_rho(t: int, tokens_per_frame: int, block_size: int, gamma: float, rho_near: float,
               rho_far: float) -> float:
    """Eq. 8: 1 for t <= 1, rho_1 when L(t) >= B_s, rho_2 otherwise (L(t) the
    unclamped Eq. 2 length, as in Eq. 11)."""
    if t <= 1:
        return 1.0
    return rho_near if decay_length(t, tokens_per_frame, gamma) >= block_size else rho_far


def static_pair_count(n_pairs: int, rho: float) -> int:
    """k = max(1, floor(|P| * rho)) in float64 (guarded, see above)."""
    return max(1, int(math.floor(float(n_pairs) * rho + COUNT_GUARD)))


def static_pair_keys(u, v, i: int, j: int, tokens_per_frame: int, seed: int) -> np.ndarray:
    """Sort keys (word << 32) | (u * N_t + v) of pairs (u, v) of frame pair (i, j)."""
    u = np.asarray(u, dtype=np.uint64)
    v = np.asarray(v, dtype=np.uint64)
    words = philox4x32_10(u, v // np.uint64(4), np.full(u.shape, i, np.uint64), np.full(u.shape, j, np.uint64),
                          seed & 0xFFFFFFFF, seed >> 32)
    lane = (v % np.uint64(4)).astype(np.int64)
    x = np.choose(lane, words)
    return (x << np.uint64(32)) | (u * np.uint64(tokens_per_frame) + v)


def static_frame_sorted_keys(i: int, j: int, tokens_per_frame: int, window: int, seed: int) -> np.ndarray:
    """Sort keys of all pairs of P(i, j) = {|u - v| <= window} (Eq. 7), ascending."""
    Nt = tokens_per_frame
    keys = []
    for u in range(Nt):
        v = np.arange(max(0, u - window), min(Nt - 1, u + window) + 1)
        keys.append(static_pair_keys(np.full(v.shape, u), v, int(i), int(j), Nt, seed))
    return np.sort(np.concatenate(keys))


def static_frame_thresholds(num_frames: int, tokens_per_frame: int, block_size: int, gamma: float, lam: float,
                            rho_near: float, rho_far: float, seed: int, query_frames=None) -> dict:
    """{(i, j): (|P|, k, largest kept sort key)} for every retained frame pair
    with t > 1 (and query frame i in query_frames, if given)."""
    Nt = tokens_per_frame
    w, sf = distance_table(num_frames, Nt, block_size, gamma, lam)
    frames = range(num_frames) if query_frames is None else query_frames
    out = {}
    for i in frames:
        for j in range(num_frames):
            t = abs(int(i) - j)
            if t <= 1 or t % sf[t] != 0:
                continue
            keys = static_frame_sorted_keys(int(i), j, Nt, w[t], seed)
            k = static_pair_count(len(keys), static_rho(t, Nt, block_size, gamma, rho_near, rho_far))
            out[(int(i), j)] = (len(keys), k, int(keys[k - 1]))
    return out


def static_selected_rows(rows: slice, num_frames: int, tokens_per_frame: int, block_size: int, gamma: float,
                         lam: float, seed: int, thresholds: dict) -> np.ndarray:
    """Selected token pairs [len(rows), S] of the query tokens `rows`: all of
    P(i, j) for t <= 1, the pairs whose sort key is at most the frame pair's
    k-th smallest for t > 1, none for frame pairs that are not retained."""
    Nt = tokens_per_frame
    w, sf = distance_table(num_frames, Nt, block_size, gamma, lam)
    S = num_frames * Nt
    sel = np.zeros((rows.stop - rows.start, S), dtype=bool)
    qtok = np.arange(rows.start, rows.stop)
    fq, uq = token_frame_and_index(qtok, Nt)
    ukey = np.arange(Nt)
    for i in np.unique(fq):
        r = np.nonzero(fq == i)[0]
        for j in range(num_frames):
            t = abs(int(i) - j)
            if t % sf[t] != 0:
                continue
            P = np.abs(uq[r][:, None] - ukey[None, :]) <= w[t]
            cols = slice(j * Nt, (j + 1) * Nt)
            if t <= 1:
                sel[r, cols] = P
                continue
            uu = np.repeat(uq[r], Nt)
            vv = np.tile(ukey, len(r))
            keys = static_pair_keys(uu, vv, int(i), j, Nt, seed).reshape(len(r), Nt)
            sel[r, cols] = P & (keys <= np.uint64(thresholds[(int(i), j)][2]))
    return sel


def static_select_rows(blocks, num_frames: int, tokens_per_frame: int, block_size: int, gamma: float, lam: float,
                       rho_near: float, rho_far: float, seed: int, theta_c: float = 0.0, theta_m: float = 0.0,
                       thresholds: dict = None) -> List[np.ndarray]:
    """Kept key blocks (ascending) of the given query blocks under the
    decay-state static-ratio mode; the mask depends on no tensor content."""
    S = num_frames * tokens_per_frame
    if thresholds is None:
        frames = sorted({f for a in blocks for f in range(a * block_size // tokens_per_frame,
                                                          (min(S, (a + 1) * block_size) - 1) // tokens_per_frame + 1)})
        thresholds = static_frame_thresholds(num_frames, tokens_per_frame, block_size, gamma, lam, rho_near,
                                             rho_far, seed, query_frames=frames)
    out = []
    for a in blocks:
        rows = slice(a * block_size, min((a + 1) * block_size, S))
        sel = static_selected_rows(rows, num_frames, tokens_per_frame, block_size, gamma, lam, seed, thresholds)
        out.append(aggregate_block_rows(sel, rows.start, block_size, S, theta_c, theta_m)[0])
    return out


def static_select(num_frames: int, tokens_per_frame: int, block_size: int, gamma: float, lam: float,
                  rho_near: float, rho_far: float, seed: int, theta_c: float = 0.0,
                  theta_m: float = 0.0) -> List[np.ndarray]:
    """Kept key blocks of every query block (ascending)."""
    S_b = -(-(num_frames * tokens_per_frame) // block_size)
    return static_select_rows(range(S_b), num_frames, tokens_per_frame, block_size, gamma, lam, rho_near,
                              rho_far, seed, theta_c, theta_m)


# ---------------------------------------------------------------------------
# 12. Proxy-task objective ([DR] App. C.2 "Mathematical Formulation of the
#     Proxy Task", C.4 "Optimization Objective", Eq. 22):
#     L(x) = ||A_dense - A_sparse(x)||_F^2 / ||A_dense||_F^2
#            + alpha * ReLU(target - S(x)),  alpha = 10, target = 0.8,
#     with A the row-softmax attention matrix (A_sparse: the softmax restricted
#     to the kept blocks, Eq. 13 with eps -> 0) and S the sparsity ratio.
#     Reading: over several heads (and batch elements) both norms are summed
#     before the ratio. The attention kernels return O = A V, not A; with V a
#     probe Z of independent N(0, 1) entries, E ||(A - A') Z||_F^2 =
#     D ||A - A'||_F^2 and E ||A Z||_F^2 = D ||A||_F^2, so the ratio of the
#     output errors estimates the normalised error of the matrices.
# ---------------------------------------------------------------------------
PROXY_ALPHA = 10.0
PROXY_TARGET = 0.8


def proxy_attention_matrices(q, k, kept, block_size: int, scale: float = None):
    """Dense and kept-block attention matrices [S, S] of one head (tiny sizes)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    S = q.shape[0]
    scale = 1.0 / math.sqrt(q.shape[1]) if scale is None else scale
    logits = (q @ k.T) * scale
    dense = _softmax_rows(logits)
    mask = np.zeros((S, S), dtype=bool)
    for a, ks in enumerate(kept):
        for b in ks:
            mask[a * block_size:min(S, (a + 1) * block_size), b * block_size:min(S, (b + 1) * block_size)] = True
    sparse = np.zeros((S, S))
    for i in range(S):
        if mask[i].any():
            sparse[i, mask[i]] = _softmax_rows(logits[i:i + 1, mask[i]])[0]
    return dense, sparse


def proxy_nmse_exact(q_heads, k_heads, kept_heads, block_size: int) -> float:
    """Eq. 22's normalised squared error of the attention matrices, summed over
    heads before the ratio."""
    num = den = 0.0
    for q, k, kept in zip(q_heads, k_heads, kept_heads):
        d, s = proxy_attention_matrices(q, k, kept, block_size)
        num += float(((d - s) ** 2).sum())
        den += float((d ** 2).sum())
    return num / den


def proxy_error_sums(q, k, z, kept, block_size: int, rows=None):
    """(sum (O_sparse - O_dense)^2, sum O_dense^2) over the given query rows
    (all by default) of one head, O = A Z."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    S = q.shape[0]
    rows = np.arange(S) if rows is None else np.asarray(rows)
    o_d = dense_attention(q, k, z, rows=rows)
    blocks = sorted({int(r) // block_size for r in rows})
    stacked = sparse_attention_rows(q, k, z, block_size, kept, blocks)   # valid rows of `blocks`, in order
    o_s = np.zeros((S, z.shape[1]))
    at = 0
    for a in blocks:
        n = min(S, (a + 1) * block_size) - a * block_size
        o_s[a * block_size:a * block_size + n] = stacked[at:at + n]
        at += n
    o_s = o_s[rows]
    return float(((o_s - o_d) ** 2).sum()), float((o_d ** 2).sum())


def proxy_sparsity(kept_heads, S_b: int) -> float:
    """1 - (kept block pairs) / (heads * S_b^2): the sparsity ratio S(x)."""
    return 1.0 - sum(len(x) for kept in kept_heads for x in kept) / float(len(kept_heads) * S_b * S_b)


def proxy_loss(nmse: float, sparsity: float, alpha: float = PROXY_ALPHA, target: float = PROXY_TARGET) -> float:
    """Eq. 22: normalised error + alpha * ReLU(target - sparsity)."""
    return nmse + alpha * max(0.0, target - sparsity)
