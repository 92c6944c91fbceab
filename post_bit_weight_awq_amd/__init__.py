"""MI355X (gfx950) AWQ per-layer search: thin Python binding of libawq_mi355x.

The functions below only marshal torch tensors into the C ABI declared in
include/awq_mi355x.h; every step of the path runs in the library's HIP
kernels on the tensors' device, on torch's current stream.  torch provides
device memory and streams, nothing else.  There is no CPU fallback: without
the built library the calls raise.

    sal = awq_act_stats(X)                          # step 1
    res = awq_search_layer(X, W, sal)               # steps 2-5: losses, i*, s*
    qweight, step, zero = awq_pack(W, res.s_best)   # codes of W diag(s*)
"""
from __future__ import annotations

import contextlib
import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import AwqConfig, AwqError, AwqSearchPlan, check, load  # noqa: F401
from ._lib import STAGE_ALL, STAGE_GRID, STAGE_PREPARE, STAGE_SELECT  # noqa: F401

__all__ = ["AwqConfig", "AwqError", "default_config", "awq_act_stats", "awq_act_stats_noalloc",
           "awq_act_stats_workspace_size", "awq_search_plan", "awq_search_workspace_size",
           "awq_search_layer", "awq_pack", "awq_w4a16_matmul", "awq_fold_inverse_scale", "awq_select_top_channels", "awq_weight_saliency",
           "SearchResult", "load"]


def default_config(n_grid: int = 20, sal_floor: float = 1e-4, *, group_size: int = 128,
                   w_bit: int = 4, zero_point: bool = True) -> AwqConfig:
    """The method's settings (4-bit, groups of 128, zero point, 20 grid points,
    floor 1e-4); the keywords select the ablation variants the library has."""
    cfg = AwqConfig()
    load().awq_default_config(ctypes.byref(cfg))
    cfg.n_grid = n_grid
    cfg.sal_floor = sal_floor
    cfg.group_size = group_size
    cfg.w_bit = w_bit
    cfg.zero_point = 1 if zero_point else 0
    return cfg


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Context in which the binding allocates its outputs and workspaces: the
    stream the kernels run on, so torch's caching allocator hands the memory
    to no other stream while they may still be pending."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, shape) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


# ------------------------------------------------------------------- stats
def awq_act_stats_workspace_size(n_tokens: int, in_features: int) -> int:
    n = load().awq_act_stats_workspace_size(n_tokens, in_features)
    if n == 0:
        raise AwqError(_lib.AWQ_ERR_INVALID_ARG, f"bad shape ({n_tokens}, {in_features})")
    return n


def awq_act_stats(X: torch.Tensor, *, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """sal[k] = mean_t |X[t, k]| as fp32, exact sum (X: [tokens, in] fp16)."""
    if X.dim() != 2:
        raise ValueError("X must be [tokens, in_features]")
    n, k = X.shape
    with _on(stream):
        if out is None:
            out = torch.empty(k, dtype=torch.float32, device=X.device)
        if workspace is None:
            workspace = torch.empty(awq_act_stats_workspace_size(n, k), dtype=torch.uint8,
                                    device=X.device)
    check(load().awq_act_stats(
        ctypes.c_void_p(_dev(X, "X", torch.float16, (n, k))), n, k,
        ctypes.c_void_p(_dev(out, "out", torch.float32, (k,))),
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


def awq_act_stats_noalloc(X: torch.Tensor, *, out: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    """The same saliency through the entry point that allocates nothing (its
    partials go to a fixed per-GPU scratch; overlapping calls on one GPU race).
    Only ``out``, when not given, is allocated here."""
    if X.dim() != 2:
        raise ValueError("X must be [tokens, in_features]")
    n, k = X.shape
    with _on(stream):
        if out is None:
            out = torch.empty(k, dtype=torch.float32, device=X.device)
    check(load().awq_act_stats_noalloc(
        ctypes.c_void_p(_dev(X, "X", torch.float16, (n, k))), n, k,
        ctypes.c_void_p(_dev(out, "out", torch.float32, (k,))), _stream(stream)))
    return out


# ------------------------------------------------------------------ search
def awq_search_plan(n_tokens: int, in_features: int, out_features: int,
                    cfg: Optional[AwqConfig] = None) -> AwqSearchPlan:
    cfg = cfg or default_config()
    plan = AwqSearchPlan()
    check(load().awq_search_plan_query(n_tokens, in_features, out_features, ctypes.byref(cfg),
                                       ctypes.byref(plan)))
    return plan


def awq_search_workspace_size(n_tokens: int, in_features: int, out_features: int,
                              cfg: Optional[AwqConfig] = None) -> int:
    return awq_search_plan(n_tokens, in_features, out_features, cfg).workspace_bytes


@dataclass
class SearchResult:
    losses: torch.Tensor     # [n_grid] float64 (device)
    best_idx: torch.Tensor   # [1] int32 (device); -1 when no loss is finite
    s_best: torch.Tensor     # [in] float32 (device)
    workspace: torch.Tensor  # uint8 workspace (tile partial sums, scale table, group parameters)
    plan: AwqSearchPlan

    def best(self) -> int:
        """The chosen grid index after synchronizing with the search's stream;
        raises AwqError(AWQ_ERR_NONFINITE) when no loss was finite."""
        b = int(self.best_idx.item())
        if b < 0:
            raise AwqError(_lib.AWQ_ERR_NONFINITE, "no grid point gave a finite loss")
        return b


def awq_search_layer(X: torch.Tensor, W: torch.Tensor, sal: torch.Tensor,
                     cfg: Optional[AwqConfig] = None, *, workspace: Optional[torch.Tensor] = None,
                     losses: Optional[torch.Tensor] = None, best_idx: Optional[torch.Tensor] = None,
                     s_best: Optional[torch.Tensor] = None, stream=None,
                     stages: int = _lib.STAGE_ALL) -> SearchResult:
    """Alpha-grid search of one layer (X: [tokens, in] fp16, W: [out, in] fp16).

    ``stages`` selects a subset of the prepare / grid / select stages (an OR
    of STAGE_PREPARE, STAGE_GRID, STAGE_SELECT); the stages of one search run
    in that order on one workspace."""
    cfg = cfg or default_config()
    if X.dim() != 2 or W.dim() != 2:
        raise ValueError("X and W must be 2-D")
    n, k = X.shape
    o = W.shape[0]
    plan = awq_search_plan(n, k, o, cfg)
    dev = X.device
    with _on(stream):
        if workspace is None:
            workspace = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
        if losses is None:
            losses = torch.empty(cfg.n_grid, dtype=torch.float64, device=dev)
        if best_idx is None:
            best_idx = torch.empty(1, dtype=torch.int32, device=dev)
        if s_best is None:
            s_best = torch.empty(k, dtype=torch.float32, device=dev)
    check(load().awq_search_layer_stages(
        stages, ctypes.c_void_p(_dev(X, "X", torch.float16, (n, k))),
        ctypes.c_void_p(_dev(W, "W", torch.float16, (o, k))),
        ctypes.c_void_p(_dev(sal, "sal", torch.float32, (k,))), n, k, o, ctypes.byref(cfg),
        ctypes.c_void_p(_dev(losses, "losses", torch.float64, (cfg.n_grid,))),
        ctypes.c_void_p(_dev(best_idx, "best_idx", torch.int32, (1,))),
        ctypes.c_void_p(_dev(s_best, "s_best", torch.float32, (k,))),
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return SearchResult(losses, best_idx, s_best, workspace, plan)


# -------------------------------------------------------------------- pack
def awq_pack(W: torch.Tensor, s: torch.Tensor, cfg: Optional[AwqConfig] = None, *,
             qweight: Optional[torch.Tensor] = None, step: Optional[torch.Tensor] = None,
             zero: Optional[torch.Tensor] = None, stream=None):
    """Codes of W diag(s): (qweight [out, in/8] int32, step [out, in/128] fp16,
    zero [out, in/128] fp16)."""
    cfg = cfg or default_config()
    if W.dim() != 2:
        raise ValueError("W must be [out_features, in_features]")
    o, k = W.shape
    g = cfg.group_size
    dev = W.device
    if k % 8 or k % g:
        raise ValueError(f"in_features={k} must be a multiple of {g}")
    with _on(stream):
        if qweight is None:
            qweight = torch.empty((o, k // 8), dtype=torch.int32, device=dev)
        if step is None:
            step = torch.empty((o, k // g), dtype=torch.float16, device=dev)
        if zero is None:
            zero = torch.empty((o, k // g), dtype=torch.float16, device=dev)
    check(load().awq_pack(
        ctypes.c_void_p(_dev(W, "W", torch.float16, (o, k))),
        ctypes.c_void_p(_dev(s, "s", torch.float32, (k,))), k, o, ctypes.byref(cfg),
        ctypes.c_void_p(_dev(qweight, "qweight", torch.int32, (o, k // 8))),
        ctypes.c_void_p(_dev(step, "step", torch.float16, (o, k // g))),
        ctypes.c_void_p(_dev(zero, "zero", torch.float16, (o, k // g))),
        _stream(stream)))
    return qweight, step, zero


def awq_w4a16_matmul(X: torch.Tensor, qweight: torch.Tensor, step: torch.Tensor,
                     zero: torch.Tensor, *, out: Optional[torch.Tensor] = None, stream=None):
    """Y [n_tokens, out_features] fp32 = X (q - zero) step, with (qweight, step,
    zero) as awq_pack returns them and X [n_tokens, in_features] fp16."""
    if X.dim() != 2 or qweight.dim() != 2:
        raise ValueError("X must be [n_tokens, in_features], qweight [out_features, in_features/8]")
    n, k = X.shape
    o = qweight.shape[0]
    if k % 128:
        raise ValueError(f"in_features={k} must be a multiple of 128")
    with _on(stream):
        if out is None:
            out = torch.empty((n, o), dtype=torch.float32, device=X.device)
    check(load().awq_w4a16_matmul(
        ctypes.c_void_p(_dev(X, "X", torch.float16, (n, k))), n, k, o,
        ctypes.c_void_p(_dev(qweight, "qweight", torch.int32, (o, k // 8))),
        ctypes.c_void_p(_dev(step, "step", torch.float16, (o, k // 128))),
        ctypes.c_void_p(_dev(zero, "zero", torch.float16, (o, k // 128))),
        ctypes.c_void_p(_dev(out, "out", torch.float32, (n, o))),
        _stream(stream)))
    return out


def awq_fold_inverse_scale(src: torch.Tensor, s: torch.Tensor, *,
                           out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Row j of the fp16 array src ([n] or [n, cols]) divided by s[j], in fp16:
    the gain or bias of the norm, or the weight or bias of the linear, that
    feeds the layer whose columns were scaled by s."""
    if src.dim() not in (1, 2):
        raise ValueError("src must be [n] or [n, cols]")
    rows = src.shape[0]
    cols = 1 if src.dim() == 1 else src.shape[1]
    with _on(stream):
        if out is None:
            out = torch.empty_like(src)
    check(load().awq_fold_inverse_scale(
        ctypes.c_void_p(_dev(src, "src", torch.float16, tuple(src.shape))),
        ctypes.c_void_p(_dev(s, "s", torch.float32, (rows,))), rows, cols,
        ctypes.c_void_p(_dev(out, "out", torch.float16, tuple(src.shape))),
        _stream(stream)))
    return out


def awq_weight_saliency(W: torch.Tensor, *, out: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """mean_o |W[o, k]| (weight-magnitude saliency): awq_act_stats over W's rows."""
    return awq_act_stats(W, out=out, stream=stream)


def awq_select_top_channels(sal: torch.Tensor, n_keep: int, *,
                            out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """sal with every channel outside the n_keep most salient set to 1."""
    if sal.dim() != 1:
        raise ValueError("sal must be [in_features]")
    n = sal.shape[0]
    with _on(stream):
        if out is None:
            out = torch.empty_like(sal)
    check(load().awq_select_top_channels(
        ctypes.c_void_p(_dev(sal, "sal", torch.float32, (n,))), n, int(n_keep),
        ctypes.c_void_p(_dev(out, "out", torch.float32, (n,))), _stream(stream)))
    return out
