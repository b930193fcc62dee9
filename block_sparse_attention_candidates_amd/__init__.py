"""DynamicRad block-sparse attention hot path for MI355X (gfx950).

Thin Python binding over libdynrad.so (include/dynrad.h). Every step of the
path runs in the library's HIP kernels; this module only checks tensor
shapes/dtypes, allocates outputs with PyTorch and passes raw device pointers
plus the current HIP stream. Method: "DynamicRad: Content-Adaptive Sparse
Attention for Long Video Diffusion" (arXiv 2604.20470).

    cand = build_candidates(radial_cfg(num_frames, tokens_per_frame, block_size, gamma, lam))
    kept = score_select(q, k, cand, mode="static", ratio=0.15)      # or mode="dynamic", tau=0.8
    out  = sparse_attn(q, k, v, cand, kept, groups="auto")       # query blocks grouped per head
    ref  = attn(q, k, v)                                            # dense baseline

q, k, v: torch.bfloat16 [B, H, S, D] contiguous CUDA (HIP) tensors,
S = num_frames * tokens_per_frame.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
from typing import Optional

import numpy as np

from . import _lib as _L
from ._lib import Dims, DynradError, RadialCfg, SelectCfg, check, lib

__all__ = ["radial_cfg", "num_blocks", "distance_table", "Candidates", "Kept", "build_candidates",
           "score_select", "token_select", "static_select", "query_groups", "query_groups_noalloc", "group_table",
           "sparse_attn", "attn", "proxy_error", "proxy_loss", "DynradError", "kept_from_lists", "wait_report",
           "set_wait_limit"]


def radial_cfg(num_frames: int, tokens_per_frame: int, block_size: int, gamma: float, lam: float,
               theta_c: float = 0.0, theta_m: float = 0.0) -> RadialCfg:
    return RadialCfg(int(num_frames), int(tokens_per_frame), int(block_size), 0, float(gamma), float(lam),
                     float(theta_c), float(theta_m))


def num_blocks(cfg: RadialCfg) -> int:
    n = lib().dr_num_blocks(ctypes.byref(cfg))
    if n < 0:
        check(int(-n))
    return int(n)


def distance_table(cfg: RadialCfg):
    """Host per-distance table (w(t), sf(t)) exactly as the candidate kernel uses it."""
    w = np.zeros(cfg.num_frames, dtype=np.int32)
    sf = np.zeros(cfg.num_frames, dtype=np.int32)
    check(lib().dr_distance_table(ctypes.byref(cfg), w.ctypes.data, sf.ctypes.data))
    return w, sf


def _torch():
    import torch
    return torch


def _stream(device):
    return ctypes.c_void_p(_torch().cuda.current_stream(device).cuda_stream)


@dataclasses.dataclass
class Candidates:
    cfg: RadialCfg
    row_ptr: "object"   # torch.int32 [S_b + 1], device
    cols: "object"      # torch.int32 [nnz], device
    nnz: int
    num_blocks: int


@dataclasses.dataclass
class Kept:
    kept_col: "object"  # torch.int32 [B * H * nnz]
    kept_cnt: "object"  # torch.int32 [B * H * S_b]
    scores: "object" = None


def build_candidates(cfg: RadialCfg, device="cuda") -> Candidates:
    torch = _torch()
    Sb = num_blocks(cfg)
    row_ptr = torch.empty(Sb + 1, dtype=torch.int32, device=device)
    cap = min(Sb * Sb, 1 << 22)
    cols = torch.empty(cap, dtype=torch.int32, device=device)
    nnz = ctypes.c_int64(0)
    st = lib().dr_build_candidates(ctypes.byref(cfg), row_ptr.data_ptr(), cols.data_ptr(), cap,
                                   ctypes.byref(nnz), _stream(row_ptr.device))
    if st == _L.DR_ERR_CAPACITY:
        cols = torch.empty(nnz.value, dtype=torch.int32, device=device)
        st = lib().dr_build_candidates(ctypes.byref(cfg), row_ptr.data_ptr(), cols.data_ptr(), nnz.value,
                                       ctypes.byref(nnz), _stream(row_ptr.device))
    check(st)
    return Candidates(cfg, row_ptr, cols[:nnz.value], int(nnz.value), Sb)


def _check_qkv(*ts):
    torch = _torch()
    shape = ts[0].shape
    for t in ts:
        if t.dtype != torch.bfloat16 or t.dim() != 4 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("q, k, v must be contiguous torch.bfloat16 CUDA tensors [B, H, S, D]")
        if t.shape != shape:
            raise ValueError("q, k, v must have the same shape")
    return shape


def _dims(shape) -> Dims:
    return Dims(int(shape[0]), int(shape[1]), int(shape[3]), 0)


def _select_cfg(mode: str, ratio: float, tau: float, score_heads: int) -> SelectCfg:
    m = {"static": _L.DR_STATIC_RATIO, "static_ratio": _L.DR_STATIC_RATIO,
         "dynamic": _L.DR_DYNAMIC_THRESHOLD, "dynamic_threshold": _L.DR_DYNAMIC_THRESHOLD}[mode]
    return SelectCfg(m, int(score_heads), float(ratio), float(tau))


def score_select(q, k, cand: Candidates, mode: str = "static", ratio: float = 1.0, tau: float = 1.0,
                 score_heads: int = 0, return_scores: bool = False, workspace=None) -> Kept:
    torch = _torch()
    shape = _check_qkv(q, k)
    if shape[2] != cand.cfg.num_frames * cand.cfg.tokens_per_frame:
        raise ValueError("sequence length does not match the candidate configuration")
    dims = _dims(shape)
    sel = _select_cfg(mode, ratio, tau, score_heads)
    B, H = int(shape[0]), int(shape[1])
    ws_bytes = ctypes.c_size_t(0)
    check(lib().dr_score_select_workspace(ctypes.byref(dims), ctypes.byref(cand.cfg), ctypes.byref(sel),
                                          cand.nnz, ctypes.byref(ws_bytes)))
    if workspace is None or workspace.numel() < ws_bytes.value:
        workspace = torch.empty(ws_bytes.value, dtype=torch.uint8, device=q.device)
    kept_col = torch.empty(B * H * cand.nnz, dtype=torch.int32, device=q.device)
    kept_cnt = torch.empty(B * H * cand.num_blocks, dtype=torch.int32, device=q.device)
    scores = None
    if return_scores:
        hm = 1 if score_heads > 0 else H
        scores = torch.empty(B * hm * cand.nnz, dtype=torch.float32, device=q.device)
    check(lib().dr_score_select(ctypes.byref(dims), ctypes.byref(cand.cfg), ctypes.byref(sel), q.data_ptr(),
                                k.data_ptr(), cand.row_ptr.data_ptr(), cand.cols.data_ptr(), cand.nnz,
                                kept_col.data_ptr(), kept_cnt.data_ptr(),
                                scores.data_ptr() if scores is not None else None,
                                workspace.data_ptr(), workspace.numel(), _stream(q.device)))
    return Kept(kept_col, kept_cnt, scores)


def token_select(q, k, cand: Candidates, tau_near: float, tau_far: float, fused_heads: int = 2,
                 eps: float = 1e-6, workspace=None) -> Kept:
    """The paper's token-level dynamic-threshold selection (dr_token_select):
    one mask per batch element from heads 0..fused_heads-1, written for every head."""
    torch = _torch()
    shape = _check_qkv(q, k)
    if shape[2] != cand.cfg.num_frames * cand.cfg.tokens_per_frame:
        raise ValueError("sequence length does not match the candidate configuration")
    dims = _dims(shape)
    tok = _L.TokenCfg(int(fused_heads), 0, float(tau_near), float(tau_far), float(eps))
    B, H = int(shape[0]), int(shape[1])
    ws_bytes = ctypes.c_size_t(0)
    check(lib().dr_token_select_workspace(ctypes.byref(dims), ctypes.byref(cand.cfg), ctypes.byref(tok),
                                          cand.nnz, ctypes.byref(ws_bytes)))
    if workspace is None or workspace.numel() < ws_bytes.value:
        workspace = torch.empty(ws_bytes.value, dtype=torch.uint8, device=q.device)
    kept_col = torch.empty(B * H * cand.nnz, dtype=torch.int32, device=q.device)
    kept_cnt = torch.empty(B * H * cand.num_blocks, dtype=torch.int32, device=q.device)
    check(lib().dr_token_select(ctypes.byref(dims), ctypes.byref(cand.cfg), ctypes.byref(tok), q.data_ptr(),
                                k.data_ptr(), cand.row_ptr.data_ptr(), cand.cols.data_ptr(), cand.nnz,
                                kept_col.data_ptr(), kept_cnt.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                _stream(q.device)))
    return Kept(kept_col, kept_cnt)


def static_select(cand: Candidates, rho_near: float, rho_far: float, seed: int, batch: int = 1, heads: int = 1,
                  workspace=None) -> Kept:
    """The paper's decay-state static-ratio selection (dr_static_select): a
    content-free mask from (rho_near, rho_far, seed), written for every one of
    batch x heads."""
    torch = _torch()
    device = cand.row_ptr.device
    dims = _L.Dims(int(batch), int(heads), 64, 0)
    st = _L.StaticCfg(float(rho_near), float(rho_far), int(seed) & 0xFFFFFFFFFFFFFFFF)
    ws_bytes = ctypes.c_size_t(0)
    check(lib().dr_static_select_workspace(ctypes.byref(cand.cfg), cand.nnz, ctypes.byref(ws_bytes)))
    if workspace is None or workspace.numel() < ws_bytes.value:
        workspace = torch.empty(ws_bytes.value, dtype=torch.uint8, device=device)
    kept_col = torch.empty(batch * heads * cand.nnz, dtype=torch.int32, device=device)
    kept_cnt = torch.empty(batch * heads * cand.num_blocks, dtype=torch.int32, device=device)
    check(lib().dr_static_select(ctypes.byref(dims), ctypes.byref(cand.cfg), ctypes.byref(st),
                                 cand.row_ptr.data_ptr(), cand.cols.data_ptr(), cand.nnz, kept_col.data_ptr(),
                                 kept_cnt.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(device)))
    return Kept(kept_col, kept_cnt)


def group_table(cand: Candidates, mode: int) -> np.ndarray:
    """Query blocks of every group of grouping mode `mode` (host; -1 = empty
    slot), shape [groups, 256 / B_s]."""
    n = lib().dr_query_group_table(ctypes.byref(cand.cfg), int(mode), None, 0)
    if n < 0:
        check(int(-n))
    t = np.empty(n, dtype=np.int32)
    m = lib().dr_query_group_table(ctypes.byref(cand.cfg), int(mode), t.ctypes.data_as(ctypes.c_void_p), n)
    if m < 0:
        check(int(-m))
    return t.reshape(-1, 256 // cand.cfg.block_size)


def query_groups(q, cand: Candidates, kept: Kept, workspace=None):
    """Per (b, h), the query-block grouping mode with the smallest total size of
    the groups' kept-list unions: torch.int32 [B * H] on q's device."""
    torch = _torch()
    dims = _dims(tuple(q.shape))
    need = ctypes.c_size_t(0)
    check(lib().dr_query_groups_workspace(ctypes.byref(dims), ctypes.byref(need)))
    if workspace is None:
        workspace = torch.empty(need.value, dtype=torch.uint8, device=q.device)
    modes = torch.empty(dims.batch * dims.heads, dtype=torch.int32, device=q.device)
    check(lib().dr_query_groups(ctypes.byref(dims), ctypes.byref(cand.cfg), cand.row_ptr.data_ptr(), cand.nnz,
                                kept.kept_col.data_ptr(), kept.kept_cnt.data_ptr(), modes.data_ptr(),
                                workspace.data_ptr(), workspace.numel(), _stream(q.device)))
    return modes


def query_groups_noalloc(q, cand: Candidates, kept: Kept, out=None):
    """query_groups without a workspace (dr_query_groups_noalloc: the library's
    per-GPU scratch array). `out`: an int32 tensor of B * H modes to fill, or
    None (then one is allocated here, by torch, outside the library)."""
    torch = _torch()
    dims = _dims(tuple(q.shape))
    modes = out if out is not None else torch.empty(dims.batch * dims.heads, dtype=torch.int32, device=q.device)
    if modes.dtype != torch.int32 or modes.numel() != dims.batch * dims.heads or not modes.is_contiguous():
        raise ValueError("out must be a contiguous int32 tensor of B * H modes")
    check(lib().dr_query_groups_noalloc(ctypes.byref(dims), ctypes.byref(cand.cfg), cand.row_ptr.data_ptr(), cand.nnz,
                                        kept.kept_col.data_ptr(), kept.kept_cnt.data_ptr(), modes.data_ptr(),
                                        _stream(q.device)))
    return modes


def sparse_attn(q, k, v, cand: Candidates, kept: Kept, softmax_scale: Optional[float] = None, out=None,
                groups=None):
    """groups: None (consecutive query blocks per workgroup), "auto" (the
    grouping chosen by query_groups) or an int32 tensor of modes [B * H].
    The output does not depend on the grouping."""
    torch = _torch()
    shape = _check_qkv(q, k, v)
    dims = _dims(shape)
    scale = 1.0 / math.sqrt(shape[3]) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if isinstance(groups, str):
        if groups != "auto":
            raise ValueError(f"groups must be None, 'auto' or a tensor, not {groups!r}")
        groups = query_groups(q, cand, kept)
    if groups is None:
        check(lib().dr_sparse_attn(ctypes.byref(dims), ctypes.byref(cand.cfg), q.data_ptr(), k.data_ptr(),
                                   v.data_ptr(), cand.row_ptr.data_ptr(), cand.nnz, kept.kept_col.data_ptr(),
                                   kept.kept_cnt.data_ptr(), scale, out.data_ptr(), _stream(q.device)))
    else:
        if groups.dtype != torch.int32 or groups.numel() != dims.batch * dims.heads or groups.device != q.device:
            raise ValueError("groups must be an int32 tensor of B * H modes on q's device")
        check(lib().dr_sparse_attn_grouped(ctypes.byref(dims), ctypes.byref(cand.cfg), q.data_ptr(), k.data_ptr(),
                                           v.data_ptr(), cand.row_ptr.data_ptr(), cand.nnz,
                                           kept.kept_col.data_ptr(), kept.kept_cnt.data_ptr(),
                                           groups.contiguous().data_ptr(), scale, out.data_ptr(),
                                           _stream(q.device)))
    return out


def attn(q, k, v, softmax_scale: Optional[float] = None, out=None):
    torch = _torch()
    shape = _check_qkv(q, k, v)
    dims = _dims(shape)
    scale = 1.0 / math.sqrt(shape[3]) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    check(lib().dr_attn(ctypes.byref(dims), int(shape[2]), q.data_ptr(), k.data_ptr(), v.data_ptr(), scale,
                        out.data_ptr(), _stream(q.device)))
    return out


def kept_from_lists(lists, row_ptr_host, batch: int, heads: int, device="cuda") -> Kept:
    """Kept-list buffers in the library layout from host lists:
    lists[(b, h)][a] = ascending key-block indices kept by query block a.
    (Used to feed any externally computed mask, e.g. a reference one.)"""
    torch = _torch()
    row_ptr_host = np.asarray(row_ptr_host, dtype=np.int64)
    Sb = len(row_ptr_host) - 1
    nnz = int(row_ptr_host[-1])
    col = np.zeros(batch * heads * nnz, dtype=np.int32)
    cnt = np.zeros(batch * heads * Sb, dtype=np.int32)
    for (b, h), rows in lists.items():
        base = (b * heads + h) * nnz
        for a, ks in enumerate(rows):
            ks = np.asarray(ks, dtype=np.int32)
            col[base + row_ptr_host[a]: base + row_ptr_host[a] + len(ks)] = ks
            cnt[(b * heads + h) * Sb + a] = len(ks)
    return Kept(torch.from_numpy(col).to(device), torch.from_numpy(cnt).to(device))


def proxy_error(o_ref, o_test, kept: Optional[Kept] = None, workspace=None):
    """dr_proxy_error: (sum (o_test - o_ref)^2, sum o_ref^2, sum of kept counts)
    over two bf16 device tensors of equal size (synchronises to read them)."""
    torch = _torch()
    if o_ref.dtype != torch.bfloat16 or o_test.dtype != torch.bfloat16 or o_ref.numel() != o_test.numel():
        raise ValueError("o_ref and o_test must be bf16 tensors of equal size")
    if not (o_ref.is_contiguous() and o_test.is_contiguous()):
        raise ValueError("o_ref and o_test must be contiguous")
    dev = o_ref.device
    out = torch.empty(3, dtype=torch.float64, device=dev)
    if workspace is None or workspace.numel() < _L.PROXY_WS_BYTES:
        workspace = torch.empty(_L.PROXY_WS_BYTES, dtype=torch.uint8, device=dev)
    cnt = kept.kept_cnt if kept is not None else None
    check(lib().dr_proxy_error(o_ref.data_ptr(), o_test.data_ptr(), o_ref.numel(),
                               cnt.data_ptr() if cnt is not None else None, cnt.numel() if cnt is not None else 0,
                               out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(dev)))
    a, b, c = out.cpu().tolist()
    return a, b, c


def proxy_loss(q, k, z, cand: Candidates, kept: Kept, alpha: float = 10.0, target: float = 0.8,
               workspace=None) -> dict:
    """The proxy-task objective of [DR] App. C.4 Eq. 22 for one mask, through
    the probe z: dense and kept-block attention of (q, k, z), then
    dr_proxy_loss forms the normalised error of the outputs, the sparsity of
    the mask and the penalised loss (synchronises to read them)."""
    torch = _torch()
    o_ref = attn(q, k, z)
    o_test = sparse_attn(q, k, z, cand, kept, groups="auto")
    dev = q.device
    B, H = int(q.shape[0]), int(q.shape[1])
    out = torch.empty(6, dtype=torch.float64, device=dev)
    if workspace is None or workspace.numel() < _L.PROXY_WS_BYTES:
        workspace = torch.empty(_L.PROXY_WS_BYTES, dtype=torch.uint8, device=dev)
    cnt = kept.kept_cnt
    check(lib().dr_proxy_loss(o_ref.data_ptr(), o_test.data_ptr(), o_ref.numel(), cnt.data_ptr(), cnt.numel(),
                              B * H * cand.num_blocks ** 2, float(alpha), float(target), out.data_ptr(),
                              workspace.data_ptr(), workspace.numel(), _stream(dev)))
    num, den, n_kept, nmse, sparsity, loss = out.cpu().tolist()
    return {"nmse": nmse, "sparsity": sparsity, "loss": loss, "err_sum": num, "ref_sum": den,
            "kept_blocks": int(n_kept)}


def wait_report(device=None) -> int:
    """dr_wait_report on the current stream of `device`: synchronises, reads
    and clears the device's flags of bounded waits that gave up; raises
    DynradError (status DR_ERR_WAIT) if any was set, else returns 0."""
    torch = _torch()
    dev = torch.device("cuda") if device is None else torch.device(device)
    flags = ctypes.c_uint32(0)
    check(lib().dr_wait_report(_stream(dev), ctypes.byref(flags)))
    return int(flags.value)


def set_wait_limit(polls: int) -> None:
    """dr_set_wait_limit: polls after which every later bounded wait gives up
    (0 restores the default). Only tests of wait_report lower it."""
    check(lib().dr_set_wait_limit(int(polls)))
