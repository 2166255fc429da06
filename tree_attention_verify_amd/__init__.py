"""MI355X (gfx950) draft-tree verify path: HIP kernels behind a C ABI.

This module is the thin Python binding of ``libtreeverify.so`` (see
``include/treeverify.h`` for the contract of every call).  It only checks
torch tensors and marshals pointers, sizes and the current HIP stream; every
step of the path runs in the library's kernels.  The library must be built
(``python -m tree_attention_verify_amd.build``); nothing here falls back to
another implementation.

Entry points (same names as the C ABI):
  tree_build_masks, tree_shift_positions, tree_attention,
  tree_attention_workspace_size, verify_tree_greedy, compact_window_rows,
  tree_sample_gumbel, tree_sample_workspace_size, tree_beam_step,
  tree_select_candidates, tree_retrieve_links, tree_attention_mla,
  tree_attention_mla_workspace_size, verify_tree_rejection,
  verify_tree_rejection_workspace_size, tree_attention_noalloc
plus verify_tree_sampled (tree_sample_gumbel, then verify_tree_greedy over
the draws).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtreeverify.so")

TAV_F32, TAV_BF16, TAV_FP8_E4M3 = 0, 1, 2
_STATUS = {0: "TAV_OK", 1: "TAV_ERR_INVALID_ARG", 2: "TAV_ERR_UNSUPPORTED",
           3: "TAV_ERR_WORKSPACE", 4: "TAV_ERR_HIP"}

# Every function the header declares.
EXPORTS = ("tav_last_error", "tav_version", "tree_build_masks", "tree_shift_positions",
           "tree_attention_workspace_size", "tree_attention", "tree_attention_prefix",
           "tree_attention_window_merge", "verify_tree_greedy", "compact_window_rows",
           "tree_sample_workspace_size", "tree_sample_gumbel", "tree_beam_step",
           "tree_select_candidates", "tree_retrieve_links", "tree_attention_mla_workspace_size",
           "tree_attention_mla", "verify_tree_rejection", "verify_tree_rejection_workspace_size",
           "tree_attention_noalloc")


class TavError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (_STATUS.get(status, status), msg))
        self.status = status


class TavRows(ctypes.Structure):
    """Mirror of the C tav_rows descriptor."""
    _fields_ = [
        ("base", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("prefix_len", ctypes.c_void_p),
        ("max_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("stride_page", ctypes.c_int64),
        ("stride_token", ctypes.c_int64),
        ("stride_head", ctypes.c_int64),
        ("stride_batch", ctypes.c_int64),
        ("n_heads", ctypes.c_int32),
        ("row_bytes", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libtreeverify.so is not built: run "
                               "`python -m tree_attention_verify_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.tav_last_error.restype = ctypes.c_char_p
        L.tav_last_error.argtypes = []
        L.tav_version.restype = ctypes.c_char_p
        L.tav_version.argtypes = []
        L.tree_build_masks.argtypes = [P, I32, I32, P, P, P, P, P, P]
        L.tree_shift_positions.argtypes = [P, P, I32, I32, I32, P]
        L.tree_attention_workspace_size.argtypes = [ctypes.c_int, I32, I32, I32, I32, I32, I32,
                                                    I32, I32]
        L.tree_attention_workspace_size.restype = ctypes.c_size_t
        attn = [P, P, P, ctypes.c_int, I64, I64, I64, I64, P, I32, I32, P, I32, I32, P, I32, I32,
                I32, I32, I32, I32, ctypes.c_float, P, P, P, ctypes.c_size_t, P]
        for f in ("tree_attention", "tree_attention_prefix", "tree_attention_window_merge"):
            getattr(L, f).argtypes = attn
            getattr(L, f).restype = ctypes.c_int
        L.tree_attention_noalloc.argtypes = attn[:24] + [P]
        L.tree_attention_noalloc.restype = ctypes.c_int
        L.verify_tree_greedy.argtypes = [P, P, P, I32, I32, P, P, P, P]
        L.compact_window_rows.argtypes = [ctypes.POINTER(TavRows), I32, P, P, I32, I32, P]
        L.tree_sample_workspace_size.argtypes = [I32, I32, I32]
        L.tree_sample_workspace_size.restype = ctypes.c_size_t
        L.tree_sample_gumbel.argtypes = [P, ctypes.c_int, I64, I32, I32, I32, P, P, P, P, P,
                                         ctypes.c_size_t, P]
        L.tree_beam_step.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, P, P, P, P, P, P]
        L.tree_select_candidates.argtypes = [P, P, P, P, I32, I32, I32, I32, P, P, P, P, P]
        L.tree_retrieve_links.argtypes = [P, I32, I32, P, P, P]
        L.tree_attention_mla_workspace_size.argtypes = [I32] * 7
        L.tree_attention_mla_workspace_size.restype = ctypes.c_size_t
        L.tree_attention_mla.argtypes = [P, P, ctypes.c_int, I64, I64, I64, P, I32, I32, P, I32,
                                         P, I32, I32, I32, I32, I32, I32, ctypes.c_float, P, P, P,
                                         ctypes.c_size_t, P]
        L.verify_tree_rejection_workspace_size.argtypes = [I32, I32, I32]
        L.verify_tree_rejection_workspace_size.restype = ctypes.c_size_t
        L.verify_tree_rejection.argtypes = [P, I64, I32, P, I64, P, P, P, P, P, I32, I32, P, P, P,
                                            P, ctypes.c_size_t, P]
        for f in ("tree_build_masks", "tree_shift_positions", "tree_attention",
                  "verify_tree_greedy", "compact_window_rows", "tree_sample_gumbel",
                  "tree_beam_step", "tree_select_candidates", "tree_retrieve_links",
                  "tree_attention_mla", "verify_tree_rejection", "verify_tree_rejection_workspace_size",
           "tree_attention_noalloc"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise TavError(status, lib().tav_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, device=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU device" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def tree_build_masks(parents: torch.Tensor, vc: Optional[torch.Tensor] = None,
                     positions: bool = True):
    """parents int32 [B][N] -> dict(depth int32, masks int64 (uint64 bits),
    positions int32 or None, tree_error int32 [B])."""
    _need(parents, "parents", torch.int32)
    B, N = parents.shape
    dev = parents.device
    depth = torch.empty((B, N), dtype=torch.int32, device=dev)
    masks = torch.empty((B, N), dtype=torch.int64, device=dev)
    err = torch.empty((B,), dtype=torch.int32, device=dev)
    pos = torch.empty((B, N), dtype=torch.int32, device=dev) if positions else None
    if vc is not None:
        _need(vc, "vc", torch.int32, dev, (B,))
    _check(lib().tree_build_masks(_ptr(parents), B, N, _ptr(vc), _ptr(depth), _ptr(masks),
                                  _ptr(pos), _ptr(err), _stream(dev)))
    return {"depth": depth, "masks": masks, "positions": pos, "tree_error": err}


def tree_shift_positions(positions: torch.Tensor, depth: torch.Tensor, direction: int):
    """In place: positions += direction * (depth - i)."""
    _need(positions, "positions", torch.int32)
    B, N = positions.shape
    _need(depth, "depth", torch.int32, positions.device, (B, N))
    _check(lib().tree_shift_positions(_ptr(positions), _ptr(depth), B, N, int(direction),
                                      _stream(positions.device)))
    return positions


def _code(q_dtype, kv_dtype=None) -> int:
    """tav_dtype of a (query, K/V cache) dtype pair."""
    kv_dtype = q_dtype if kv_dtype is None else kv_dtype
    if q_dtype == torch.bfloat16 and kv_dtype == torch.float8_e4m3fn:
        return TAV_FP8_E4M3
    if q_dtype != kv_dtype:
        raise TypeError("K/V caches must have q's dtype, or be float8_e4m3fn under a bf16 q")
    if q_dtype == torch.bfloat16:
        return TAV_BF16
    if q_dtype == torch.float32:
        return TAV_F32
    raise TypeError("q must be float32 or bfloat16, got %s" % q_dtype)


def tree_attention_workspace_size(dtype, B, R, Hq, Hkv, D, max_prefix_len, prefix_window,
                                  page_size, kv_dtype=None) -> int:
    code = _code(dtype, kv_dtype)
    return int(lib().tree_attention_workspace_size(code, B, R, Hq, Hkv, D, max_prefix_len,
                                                   prefix_window, page_size))


def kv_strides(cache: torch.Tensor, layout: str):
    """(page, head, token) element strides of a 4-D paged cache."""
    if cache.dim() != 4 or cache.stride(3) != 1:
        raise ValueError("K/V caches must be 4-D with contiguous channels")
    if layout == "HND":      # [pages][Hkv][page_size][D]
        return cache.stride(0), cache.stride(1), cache.stride(2), cache.shape[1], cache.shape[2]
    if layout == "NHD":      # [pages][page_size][Hkv][D]
        return cache.stride(0), cache.stride(2), cache.stride(1), cache.shape[2], cache.shape[1]
    raise ValueError("layout must be 'HND' or 'NHD'")


def tree_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   page_table: torch.Tensor, prefix_len: torch.Tensor, masks: torch.Tensor,
                   W: int, *, max_prefix_len: int, layout: str = "HND", prefix_window: int = 0,
                   sm_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                   lse2: Optional[torch.Tensor] = None, return_lse: bool = True,
                   workspace: Optional[torch.Tensor] = None, phase: str = "all"):
    """Tree attention (see include/treeverify.h).  q [B][R][Hq][D] fp32/bf16;
    k_cache/v_cache paged pools in `layout`, of q's dtype or float8_e4m3fn
    under a bf16 q; page_table int32 [B][max_pages];
    prefix_len int32 [B]; masks int64 [B][R] (uint64 bit patterns).
    phase: "all" (tree_attention), "prefix" (tree_attention_prefix) or
    "window_merge" (tree_attention_window_merge; pass the workspace, out
    and lse2 of the prefix phase: with a single split the prefix phase may
    write the output itself).
    Returns (out [B][R][Hq][D], lse2 float32 [B][R][Hq] or None)."""
    fn = {"all": "tree_attention", "prefix": "tree_attention_prefix",
          "window_merge": "tree_attention_window_merge"}[phase]
    if phase == "window_merge" and (out is None or workspace is None or
                                    (return_lse and lse2 is None)):
        raise ValueError("phase='window_merge' takes the workspace, out and lse2 "
                         "of the prefix phase")
    dt = _code(q.dtype, k_cache.dtype)
    _need(q, "q", q.dtype)
    dev = q.device
    B, R, Hq, D = q.shape
    _need(k_cache, "k_cache", k_cache.dtype, dev)
    _need(v_cache, "v_cache", k_cache.dtype, dev)
    sp, sh, st, Hkv, ps = kv_strides(k_cache, layout)
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("v_cache must have k_cache's shape")
    _need(page_table, "page_table", torch.int32, dev)
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be [B][max_pages]")
    _need(prefix_len, "prefix_len", torch.int32, dev, (B,))
    _need(masks, "masks", torch.int64, dev, (B, R))
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", q.dtype, dev, q.shape)
    if lse2 is None and return_lse:
        lse2 = torch.empty((B, R, Hq), dtype=torch.float32, device=dev)
    elif lse2 is not None:
        _need(lse2, "lse2", torch.float32, dev, (B, R, Hq))
    need = lib().tree_attention_workspace_size(dt, B, R, Hq, Hkv, D, max_prefix_len,
                                               prefix_window, ps)
    if workspace is None:
        workspace = torch.empty(max(int(need), 256), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", torch.uint8, dev)
    _check(getattr(lib(), fn)(_ptr(q), _ptr(k_cache), _ptr(v_cache), dt, sp, sh, st,
                                k_cache.shape[0], _ptr(page_table), page_table.shape[1], ps,
                                _ptr(prefix_len), int(max_prefix_len), int(prefix_window),
                                _ptr(masks), int(W), B, R, Hq, Hkv, D, float(sm_scale),
                                _ptr(out), _ptr(lse2), _ptr(workspace), workspace.numel(),
                                _stream(dev)))
    return out, lse2


NOALLOC_SCRATCH_BYTES = 64 << 20   # TAV_NOALLOC_SCRATCH_BYTES


def tree_attention_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           page_table: torch.Tensor, prefix_len: torch.Tensor,
                           masks: torch.Tensor, W: int, *, max_prefix_len: int, out: torch.Tensor,
                           lse2: Optional[torch.Tensor] = None, layout: str = "HND",
                           prefix_window: int = 0, sm_scale: float = 0.0):
    """tree_attention with its partials in the library's fixed device array
    (no workspace, nothing allocated here or in the library: the caller
    passes out, and lse2 or None).  Calls that overlap on one GPU race.
    Returns (out, lse2)."""
    dt = _code(q.dtype, k_cache.dtype)
    _need(q, "q", q.dtype)
    dev = q.device
    B, R, Hq, D = q.shape
    _need(k_cache, "k_cache", k_cache.dtype, dev)
    _need(v_cache, "v_cache", k_cache.dtype, dev)
    sp, sh, st, Hkv, ps = kv_strides(k_cache, layout)
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("v_cache must have k_cache's shape")
    _need(page_table, "page_table", torch.int32, dev)
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be [B][max_pages]")
    _need(prefix_len, "prefix_len", torch.int32, dev, (B,))
    _need(masks, "masks", torch.int64, dev, (B, R))
    _need(out, "out", q.dtype, dev, q.shape)
    if lse2 is not None:
        _need(lse2, "lse2", torch.float32, dev, (B, R, Hq))
    _check(lib().tree_attention_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), dt, sp, sh, st,
                                        k_cache.shape[0], _ptr(page_table), page_table.shape[1],
                                        ps, _ptr(prefix_len), int(max_prefix_len),
                                        int(prefix_window), _ptr(masks), int(W), B, R, Hq, Hkv, D,
                                        float(sm_scale), _ptr(out), _ptr(lse2), _stream(dev)))
    return out, lse2


def verify_tree_greedy(draft_tokens: torch.Tensor, target_argmax: torch.Tensor,
                       parents: torch.Tensor, tokens: bool = True):
    """-> dict(accepted_path int32 [B][N], accept_len int32 [B],
    accepted_tokens int32 [B][N] or None)."""
    _need(parents, "parents", torch.int32)
    B, N = parents.shape
    dev = parents.device
    _need(draft_tokens, "draft_tokens", torch.int32, dev, (B, N))
    _need(target_argmax, "target_argmax", torch.int32, dev, (B, N))
    path = torch.empty((B, N), dtype=torch.int32, device=dev)
    alen = torch.empty((B,), dtype=torch.int32, device=dev)
    tok = torch.empty((B, N), dtype=torch.int32, device=dev) if tokens else None
    _check(lib().verify_tree_greedy(_ptr(draft_tokens), _ptr(target_argmax), _ptr(parents), B, N,
                                    _ptr(path), _ptr(alen), _ptr(tok), _stream(dev)))
    return {"accepted_path": path, "accept_len": alen, "accepted_tokens": tok}


def tree_sample_workspace_size(B: int, N: int, V: int) -> int:
    return int(lib().tree_sample_workspace_size(B, N, V))


def tree_sample_gumbel(logits: torch.Tensor, temperature: torch.Tensor, seed: torch.Tensor,
                       positions: torch.Tensor, workspace: Optional[torch.Tensor] = None):
    """Gumbel-max target draw of every verify row, keyed by (seed[b],
    positions[b][i] + 1).

    logits bf16 or float32 [B][N][V] (rows may be padded: the last dim's
    stride must span a multiple of 16 bytes); temperature float32 [B] (<= 0:
    greedy argmax); seed int64 [B] (the uint64 seed's bits); positions int32
    [B][N] (vc + depth).  -> tokens int32 [B][N]."""
    if logits.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("logits must be bfloat16 or float32, got %s" % logits.dtype)
    if not logits.is_cuda or logits.dim() != 3 or logits.stride(2) != 1 \
            or logits.stride(0) != logits.shape[1] * logits.stride(1):
        raise ValueError("logits must be a [B][N][V] GPU tensor with unit channel stride and "
                         "rows at a constant stride")
    B, N, V = logits.shape
    dev = logits.device
    _need(temperature, "temperature", torch.float32, dev, (B,))
    _need(seed, "seed", torch.int64, dev, (B,))
    _need(positions, "positions", torch.int32, dev, (B, N))
    need = tree_sample_workspace_size(B, N, V)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    dt = TAV_BF16 if logits.dtype == torch.bfloat16 else TAV_F32
    _check(lib().tree_sample_gumbel(_ptr(logits), dt, logits.stride(1), V, B, N, _ptr(temperature),
                                    _ptr(seed), _ptr(positions), _ptr(tokens), _ptr(workspace),
                                    workspace.numel(), _stream(dev)))
    return tokens


def verify_tree_sampled(draft_tokens: torch.Tensor, logits: torch.Tensor,
                        temperature: torch.Tensor, seed: torch.Tensor, positions: torch.Tensor,
                        parents: torch.Tensor, workspace: Optional[torch.Tensor] = None):
    """Sampled verify: the Gumbel-max draws of every row, then the greedy
    tree walk over them.  -> dict(draws, accepted_path, accept_len,
    accepted_tokens)."""
    draws = tree_sample_gumbel(logits, temperature, seed, positions, workspace)
    r = verify_tree_greedy(draft_tokens, draws, parents)
    r["draws"] = draws
    return r


def verify_tree_rejection(probs: torch.Tensor, draft_tokens: torch.Tensor, parents: torch.Tensor,
                          coins: torch.Tensor, bonus_u: torch.Tensor,
                          draft_score: Optional[torch.Tensor] = None, tokens: bool = True,
                          draft_q: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None):
    """Tree rejection sampling: probs float32 [B][N][V] (the target
    distribution after every node; rows may be padded to a stride of a
    multiple of 4), draft_tokens / parents int32 [B][N], coins / bonus_u
    float32 [B][N] uniform in [0, 1), draft_score float32 [B][N] or None
    (the sibling order), draft_q float32 [B][N][V] or None (the draft
    distribution that drew each node's children: test against it),
    workspace uint8 of >= verify_tree_rejection_workspace_size(B, N, V)
    bytes or None (allocated here).
    -> dict(accepted_path, accept_len, accepted_tokens)."""
    if probs.dtype != torch.float32 or not probs.is_cuda or probs.dim() != 3 \
            or probs.stride(2) != 1 or probs.stride(0) != probs.shape[1] * probs.stride(1):
        raise ValueError("probs must be a float32 [B][N][V] GPU tensor with unit channel stride "
                         "and rows at a constant stride")
    B, N, V = probs.shape
    dev = probs.device
    _need(draft_tokens, "draft_tokens", torch.int32, dev, (B, N))
    _need(parents, "parents", torch.int32, dev, (B, N))
    _need(coins, "coins", torch.float32, dev, (B, N))
    _need(bonus_u, "bonus_u", torch.float32, dev, (B, N))
    if draft_score is not None:
        _need(draft_score, "draft_score", torch.float32, dev, (B, N))
    qs = 0
    if draft_q is not None:
        if draft_q.dtype != torch.float32 or draft_q.device != dev or draft_q.dim() != 3 \
                or tuple(draft_q.shape) != (B, N, V) or draft_q.stride(2) != 1 \
                or draft_q.stride(0) != N * draft_q.stride(1):
            raise ValueError("draft_q must be a float32 [B][N][V] tensor on the device of probs "
                             "with unit channel stride and rows at a constant stride")
        qs = draft_q.stride(1)
    path = torch.empty((B, N), dtype=torch.int32, device=dev)
    alen = torch.empty((B,), dtype=torch.int32, device=dev)
    tok = torch.empty((B, N), dtype=torch.int32, device=dev) if tokens else None
    need = verify_tree_rejection_workspace_size(B, N, V)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    _check(lib().verify_tree_rejection(_ptr(probs), probs.stride(1), V, _ptr(draft_q), qs,
                                       _ptr(draft_tokens),
                                       _ptr(parents), _ptr(draft_score), _ptr(coins),
                                       _ptr(bonus_u), B, N, _ptr(path), _ptr(alen), _ptr(tok),
                                       _ptr(workspace), workspace.numel(), _stream(dev)))
    return {"accepted_path": path, "accept_len": alen, "accepted_tokens": tok}


def verify_tree_rejection_workspace_size(B: int, N: int, V: int) -> int:
    return int(lib().verify_tree_rejection_workspace_size(B, N, V))


def tree_attention_mla_workspace_size(B: int, R: int, Hq: int, Dc: int, Dr: int,
                                      max_prefix_len: int, page_size: int) -> int:
    return int(lib().tree_attention_mla_workspace_size(B, R, Hq, Dc, Dr, max_prefix_len,
                                                       page_size))


def tree_attention_mla(q: torch.Tensor, latent: torch.Tensor, page_table: torch.Tensor,
                       prefix_len: torch.Tensor, masks: torch.Tensor, W: int, Dc: int = 512, *,
                       max_prefix_len: int, sm_scale: float = 0.0,
                       workspace: Optional[torch.Tensor] = None):
    """Tree attention over an MLA latent cache.  q bf16 [B][R][Hq][Dc + Dr];
    latent bf16 or float8_e4m3fn [pages][page_size][Dc + Dr] (under an E4M3
    cache every key is scored with q rounded to E4M3); page_table int32 [B][max_pages];
    prefix_len int32 [B]; masks int64 (uint64 bits) [B][R].  max_prefix_len
    (a host int >= every prefix_len) sizes the workspace and the split plan;
    it is required, as for tree_attention, so the call never reads the device.
    -> (out bf16 [B][R][Hq][Dc], lse2 float32 [B][R][Hq])."""
    _need(q, "q", torch.bfloat16)
    B, R, Hq, Dk = q.shape
    Dr = Dk - Dc
    dev = q.device
    if latent.dtype == torch.float8_e4m3fn:
        _need(latent, "latent", torch.float8_e4m3fn, dev)
        lat_code = TAV_FP8_E4M3
    else:
        _need(latent, "latent", torch.bfloat16, dev)
        lat_code = TAV_BF16
    if latent.dim() != 3 or latent.shape[2] != Dk:
        raise ValueError("latent must be [pages][page_size][Dc + Dr]")
    pages, ps = latent.shape[0], latent.shape[1]
    _need(page_table, "page_table", torch.int32, dev)
    _need(prefix_len, "prefix_len", torch.int32, dev, (B,))
    _need(masks, "masks", torch.int64, dev, (B, R))
    need = tree_attention_mla_workspace_size(B, R, Hq, Dc, Dr, max_prefix_len, ps)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    out = torch.empty((B, R, Hq, Dc), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, R, Hq), dtype=torch.float32, device=dev)
    _check(lib().tree_attention_mla(_ptr(q), _ptr(latent), lat_code, ps * Dk, Dk, pages,
                                    _ptr(page_table), page_table.shape[1], ps, _ptr(prefix_len),
                                    int(max_prefix_len), _ptr(masks), int(W), B, R, Hq, Dc, Dr,
                                    float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                    workspace.numel(), _stream(dev)))
    return out, lse


def tree_beam_step(scores: torch.Tensor, surv_idx: torch.Tensor, child_p: torch.Tensor,
                   child_tok: torch.Tensor, pool_scores: torch.Tensor, pool_parents: torch.Tensor,
                   pool_tokens: torch.Tensor, pool_base: int):
    """One EAGLE-2 expansion: writes the step's pool entries in place and
    returns (next_scores float32 [B][K], next_idx int32 [B][K])."""
    _need(child_p, "child_p", torch.float32)
    B, S, K = child_p.shape
    dev = child_p.device
    _need(scores, "scores", torch.float32, dev, (B, S))
    _need(surv_idx, "surv_idx", torch.int32, dev, (B, S))
    _need(child_tok, "child_tok", torch.int32, dev, (B, S, K))
    _need(pool_scores, "pool_scores", torch.float32, dev)
    C = pool_scores.shape[1]
    _need(pool_parents, "pool_parents", torch.int32, dev, (B, C))
    _need(pool_tokens, "pool_tokens", torch.int32, dev, (B, C))
    ns = torch.empty((B, K), dtype=torch.float32, device=dev)
    ni = torch.empty((B, K), dtype=torch.int32, device=dev)
    _check(lib().tree_beam_step(_ptr(scores), _ptr(surv_idx), _ptr(child_p), _ptr(child_tok), B, S,
                                K, C, int(pool_base), _ptr(pool_scores), _ptr(pool_parents),
                                _ptr(pool_tokens), _ptr(ns), _ptr(ni), _stream(dev)))
    return ns, ni


def tree_select_candidates(pool_scores: torch.Tensor, pool_parents: torch.Tensor,
                           pool_tokens: torch.Tensor, root_tokens: torch.Tensor, N: int,
                           order: int = 0):
    """The verify tree from the candidate pool.  -> dict(parents, tokens,
    selected int32 [B][N], tree_error int32 [B])."""
    _need(pool_scores, "pool_scores", torch.float32)
    B, C = pool_scores.shape
    dev = pool_scores.device
    _need(pool_parents, "pool_parents", torch.int32, dev, (B, C))
    _need(pool_tokens, "pool_tokens", torch.int32, dev, (B, C))
    _need(root_tokens, "root_tokens", torch.int32, dev, (B,))
    out = {k: torch.empty((B, N), dtype=torch.int32, device=dev)
           for k in ("parents", "tokens", "selected")}
    out["tree_error"] = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(lib().tree_select_candidates(_ptr(pool_scores), _ptr(pool_parents), _ptr(pool_tokens),
                                        _ptr(root_tokens), B, C, int(N), int(order),
                                        _ptr(out["parents"]), _ptr(out["tokens"]),
                                        _ptr(out["selected"]), _ptr(out["tree_error"]),
                                        _stream(dev)))
    return out


def tree_retrieve_links(parents: torch.Tensor):
    """-> (next_token, next_sibling) int32 [B][N]."""
    _need(parents, "parents", torch.int32)
    B, N = parents.shape
    dev = parents.device
    nt = torch.empty((B, N), dtype=torch.int32, device=dev)
    ns = torch.empty((B, N), dtype=torch.int32, device=dev)
    _check(lib().tree_retrieve_links(_ptr(parents), B, N, _ptr(nt), _ptr(ns), _stream(dev)))
    return nt, ns


@dataclasses.dataclass
class RowTable:
    """One buffer for compact_window_rows (byte strides; see tav_rows)."""
    buf: torch.Tensor
    row_bytes: int
    stride_token: int
    n_heads: int = 1
    stride_head: int = 0
    stride_batch: int = 0
    page_table: Optional[torch.Tensor] = None
    prefix_len: Optional[torch.Tensor] = None
    page_size: int = 1
    stride_page: int = 0
    num_pages: int = 0

    @staticmethod
    def paged_kv(cache: torch.Tensor, page_table: torch.Tensor, prefix_len: torch.Tensor,
                 layout: str = "HND") -> "RowTable":
        sp, sh, st, Hkv, ps = kv_strides(cache, layout)
        e = cache.element_size()
        return RowTable(buf=cache, row_bytes=cache.shape[3] * e, stride_token=st * e,
                        n_heads=Hkv, stride_head=sh * e, page_table=page_table,
                        prefix_len=prefix_len, page_size=ps, stride_page=sp * e,
                        num_pages=cache.shape[0])

    @staticmethod
    def dense_rows(rows: torch.Tensor) -> "RowTable":
        """rows [B][N][...]: one row of prod(...) elements per window slot."""
        e = rows.element_size()
        per = rows[0, 0].numel() * e
        return RowTable(buf=rows, row_bytes=per, stride_token=rows.stride(1) * e,
                        stride_batch=rows.stride(0) * e)


def compact_window_rows(tables: Sequence[RowTable], accepted_path: torch.Tensor,
                        accept_len: torch.Tensor):
    """Moves each request's accepted rows to the window's leading slots, in
    place, in every table."""
    _need(accepted_path, "accepted_path", torch.int32)
    B, N = accepted_path.shape
    dev = accepted_path.device
    _need(accept_len, "accept_len", torch.int32, dev, (B,))
    arr = (TavRows * max(1, len(tables)))()
    for i, t in enumerate(tables):
        if not t.buf.is_cuda or t.buf.device != dev:
            raise ValueError("table %d buffer must be on %s" % (i, dev))
        if t.page_table is not None:
            _need(t.page_table, "page_table", torch.int32, dev)
            _need(t.prefix_len, "prefix_len", torch.int32, dev, (B,))
        arr[i] = TavRows(t.buf.data_ptr(), _ptr(t.page_table), _ptr(t.prefix_len),
                         0 if t.page_table is None else t.page_table.shape[1], int(t.page_size),
                         int(t.num_pages), int(t.stride_page), int(t.stride_token),
                         int(t.stride_head), int(t.stride_batch), int(t.n_heads),
                         int(t.row_bytes))
    _check(lib().compact_window_rows(arr, len(tables), _ptr(accepted_path), _ptr(accept_len), B,
                                     N, _stream(dev)))
