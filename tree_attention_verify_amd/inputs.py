"""Seeded synthetic inputs for the draft-tree verify path.

This module only draws inputs: random trees, draft/target tokens, query and
paged K/V tensors, page tables and lane masks.  It computes none of the
method's results (no ancestor masks of a verify tree, no attention, no walk,
no compaction), so the HIP path and the oracle can both take their inputs
from here without sharing arithmetic.

Workloads (the shapes of the five synthetic verify configurations):

  worked   B 1, P 128, N 5 [root, A, B, C, D], parents [-1, 0, 0, 1, 2],
           Hq 4, Hkv 1, D 64, fp32, page size 16
  random16 B 8, P 2048, N 16 random trees (depth <= 6), Hq 32, Hkv 8, D 128,
           bf16, page size 16
  eagle64  B 32, P 8192, EAGLE-style top-8 beam over 6 expansion steps, best 63
           plus root (N 64), Hq 64, Hkv 8, D 128, bf16, page size 16
  long64   B 4, P 131072, N 64 random trees (depth <= 8), Hq 32, Hkv 8, D 128,
           bf16, page size 64
  lanes    B 64, P 32768, draft lanes K 4 over S 4 steps (R 4, W 12), frozen
           4096-key sliding window, Hq 32, Hkv 8, D 128, bf16, page size 16
  chain8   B 64, P 32768, chain tree N 8 (parent[i] = i - 1), same shapes
  long64_tp8  long64 at one 8-way tensor-parallel share: Hq 4, Hkv 1

Recipe: tree structure and tokens come from numpy PCG64 streams spawned from
SeedSequence(seed); tensors from a torch generator seeded from the same
SeedSequence on the device they are made on.  q/k/v are N(0, 1) drawn in fp32
and rounded to bf16 (round-to-nearest-even) except for fp32 workloads.  The
page pool has 1 + B * pages_per_request pages; page 0 is never referenced and
is NaN-filled, and every slot past a request's prefix + window is NaN, so any
read of an unseen slot shows up in the outputs.  The page table is a seeded
permutation of pages 1..pool-1.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

VOCAB = 1000


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    P: int
    N: int          # verify nodes (tree workloads) or lane rows (lanes)
    Hq: int
    Hkv: int
    D: int
    dtype: str      # "f32" | "bf16"
    page_size: int
    tree: str       # "worked" | "random" | "eagle" | "chain" | "lanes"
    depth_cap: int = 0
    prefix_window: int = 0
    lane_k: int = 0
    lane_steps: int = 0
    eagle_topk: int = 0
    eagle_steps: int = 0
    kv_dtype: str = ""  # K/V cache dtype when it differs from dtype: "fp8" (E4M3, bf16 q)

    @property
    def kv(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def R(self) -> int:
        return self.lane_k if self.tree == "lanes" else self.N

    @property
    def W(self) -> int:
        return (self.lane_steps - 1) * self.lane_k if self.tree == "lanes" else self.N

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def describe(self) -> str:
        tree = {
            "worked": "the worked 5-node tree [root, A, B, C, D]",
            "random": "N %d random trees (depth <= %d)" % (self.N, self.depth_cap),
            "eagle": "EAGLE beam trees (top-%d, %d steps, best %d nodes + root)"
                     % (self.eagle_topk, self.eagle_steps, self.N - 1),
            "chain": "a chain of N %d" % self.N,
            "lanes": "draft lanes (K %d, S %d, W %d) over a frozen %d-key window"
                     % (self.lane_k, self.lane_steps, self.W, self.prefix_window),
        }[self.tree]
        dt = self.dtype if self.kv == self.dtype else "%s q, %s E4M3 K/V" % (self.dtype, self.kv)
        return "%s: B %d, P %d, %s, Hq %d, Hkv %d, D %d, %s, page size %d" % (
            self.name, self.B, self.P, tree, self.Hq, self.Hkv, self.D, dt, self.page_size)


WORKLOADS = {
    "worked": Workload("worked", 1, 128, 5, 4, 1, 64, "f32", 16, "worked"),
    "random16": Workload("random16", 8, 2048, 16, 32, 8, 128, "bf16", 16, "random",
                         depth_cap=6),
    "eagle64": Workload("eagle64", 32, 8192, 64, 64, 8, 128, "bf16", 16, "eagle",
                        eagle_topk=8, eagle_steps=6),
    "long64": Workload("long64", 4, 131072, 64, 32, 8, 128, "bf16", 64, "random",
                       depth_cap=8),
    "lanes": Workload("lanes", 64, 32768, 4, 32, 8, 128, "bf16", 16, "lanes",
                      prefix_window=4096, lane_k=4, lane_steps=4),
    "chain8": Workload("chain8", 64, 32768, 8, 32, 8, 128, "bf16", 16, "chain"),
    # the long-context workload over an FP8 E4M3 K/V cache (bf16 query and output)
    "long64_fp8": Workload("long64_fp8", 4, 131072, 64, 32, 8, 128, "bf16", 64, "random",
                           depth_cap=8, kv_dtype="fp8"),
    "chain8_fp8": Workload("chain8_fp8", 64, 32768, 8, 32, 8, 128, "bf16", 16, "chain",
                           kv_dtype="fp8"),
    # one tensor-parallel share of long64 over 8 GPUs: each GPU holds one kv
    # head and its 4 query heads, with the same trees and prefix
    "long64_tp8": Workload("long64_tp8", 4, 131072, 64, 4, 1, 128, "bf16", 64, "random",
                           depth_cap=8),
}


def _streams(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def _torch_seed(seed: int, k: int) -> int:
    return int(np.random.SeedSequence([seed, 7919, k]).generate_state(1, dtype=np.uint64)[0] >> 1)


# ---------------------------------------------------------------------------
# tree structure
# ---------------------------------------------------------------------------

def random_tree(rng, N: int, depth_cap: int) -> np.ndarray:
    """Node 0 is the root; node i > 0 picks its parent uniformly among earlier
    nodes whose depth is below depth_cap (so no node is deeper than the cap)."""
    par = np.full(N, -1, np.int32)
    lvl = np.zeros(N, np.int32)   # generation bookkeeping for the cap
    for i in range(1, N):
        ok = np.nonzero(lvl[:i] < depth_cap)[0]
        p = int(ok[rng.integers(0, ok.size)])
        par[i] = p
        lvl[i] = lvl[p] + 1
    return par


def chain_tree(N: int) -> np.ndarray:
    return np.arange(-1, N - 1, dtype=np.int32)


def eagle_tree(rng, topk: int, steps: int, N: int) -> np.ndarray:
    """EAGLE-2 style beam: the root expands into topk children; at each later
    step the topk best candidates of the previous step's expansion each expand
    into topk children.  Child probabilities are Dirichlet(1) per parent and a
    candidate's score is the product along its path (fp64).  The N - 1 best
    candidates by (-score, pool index) are kept, sorted by pool index, and the
    root is prepended as node 0.  Parents precede children in pool order and
    scores shrink along a path, so every kept node's parent is kept too."""
    pool_parent = []   # parent pool index (-1 = root)
    pool_score = []
    frontier = [(-1, 1.0)]  # (pool index, score) of the nodes expanded next
    for _ in range(steps):
        cand = []
        for (pidx, pscore) in frontier:
            probs = rng.dirichlet(np.ones(topk))
            for c in range(topk):
                idx = len(pool_parent)
                pool_parent.append(pidx)
                pool_score.append(pscore * float(probs[c]))
                cand.append(idx)
        order = sorted(cand, key=lambda i: (-pool_score[i], i))
        frontier = [(i, pool_score[i]) for i in order[:topk]]
    order = sorted(range(len(pool_parent)), key=lambda i: (-pool_score[i], i))
    keep = sorted(order[:N - 1])
    node_of = {p: n + 1 for n, p in enumerate(keep)}
    par = np.full(N, -1, np.int32)
    for n, p in enumerate(keep):
        pp = pool_parent[p]
        par[n + 1] = 0 if pp == -1 else node_of[pp]   # closure: KeyError if broken
    return par


def lane_masks(rng, B: int, K: int, S: int) -> tuple[np.ndarray, np.ndarray]:
    """Draft-lane window of (S - 1) * K keys: lane r of step s (1-based) owns
    key (s - 1) * K + r and follows a parent lane of step s - 1 chosen
    uniformly; step-1 lanes hang off the committed frontier.  Returns the lane
    parents (-1 for step 1) and the drafter-side ancestor masks of the last
    step's K lane rows, which are what the lane attention reads."""
    W = (S - 1) * K
    par = np.full((B, W), -1, np.int32)
    masks = np.zeros((B, K), np.uint64)
    for b in range(B):
        own = [np.uint64(0)] * W
        for key in range(W):
            step = key // K
            m = np.uint64(1) << np.uint64(key)
            if step > 0:
                p = (step - 1) * K + int(rng.integers(0, K))
                par[b, key] = p
                m |= own[p]
            own[key] = m
        masks[b] = own[W - K:]
    return par, masks


def tokens_for(rng, parents: np.ndarray, agree: Optional[float]) -> tuple[np.ndarray, np.ndarray]:
    """Draft tokens and target argmax per node.  Siblings get distinct draft
    tokens.  With agree = p: for a node with children, the target token is a
    uniformly chosen child's draft token with probability p, else a token none
    of its children carries; leaves get a random token.  agree=None draws both
    uniformly in [0, VOCAB)."""
    N = parents.size
    if agree is None:
        return (rng.integers(0, VOCAB, N).astype(np.int32),
                rng.integers(0, VOCAB, N).astype(np.int32))
    children = [[] for _ in range(N)]
    for i in range(1, N):
        if 0 <= parents[i] < N:
            children[parents[i]].append(i)
    draft = np.zeros(N, np.int32)
    draft[0] = rng.integers(0, VOCAB)
    for v in range(N):
        if children[v]:
            draft[children[v]] = rng.choice(VOCAB, size=len(children[v]), replace=False)
    target = np.zeros(N, np.int32)
    for v in range(N):
        ch = children[v]
        if ch and rng.random() < agree:
            target[v] = draft[ch[rng.integers(0, len(ch))]]
        else:
            used = set(int(draft[c]) for c in ch)
            t = int(rng.integers(0, VOCAB))
            while t in used:
                t = int(rng.integers(0, VOCAB))
            target[v] = t
    return draft, target


# ---------------------------------------------------------------------------
# tensors
# ---------------------------------------------------------------------------

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


def _randn_into(out: torch.Tensor, gen: torch.Generator, chunk: int = 1 << 26):
    flat = out.view(-1)
    for s in range(0, flat.numel(), chunk):
        e = min(flat.numel(), s + chunk)
        flat[s:e] = torch.randn(e - s, generator=gen, device=out.device,
                                dtype=torch.float32).to(out.dtype)


@dataclasses.dataclass
class Inputs:
    wl: Workload
    parents: np.ndarray          # [B][N] int32 (lanes: [B][W] lane parents)
    draft: np.ndarray            # [B][N] int32
    target: np.ndarray           # [B][N] int32
    lane_masks: Optional[np.ndarray]  # [B][R] uint64 (lanes only)
    prefix_len: np.ndarray       # [B] int32
    page_table: np.ndarray       # [B][max_pages] int32
    q: torch.Tensor              # [B][R][Hq][D]
    k_cache: torch.Tensor        # [pages][Hkv][ps][D] (HND) or [pages][ps][Hkv][D] (NHD)
    v_cache: torch.Tensor
    layout: str                  # "HND" | "NHD"

    @property
    def strides(self):
        """(page, head, token) strides in elements."""
        wl = self.wl
        if self.layout == "HND":
            return (wl.Hkv * wl.page_size * wl.D, wl.page_size * wl.D, wl.D)
        return (wl.page_size * wl.Hkv * wl.D, wl.D, wl.Hkv * wl.D)


def make_inputs(wl: Workload, seed: int, device="cpu", layout: str = "HND",
                prefix_lens: Optional[np.ndarray] = None, with_tensors: bool = True) -> Inputs:
    """All inputs of one step of the workload, seeded.  prefix_lens overrides
    the per-request prefix length (ragged batches); pages per request cover
    max(prefix) + W."""
    r_tree, r_tok, r_pt, r_lane = _streams(seed, 4)
    B, N = wl.B, wl.N
    lm = None
    if wl.tree == "lanes":
        parents, lm = lane_masks(r_lane, B, wl.lane_k, wl.lane_steps)
        draft = np.zeros((B, wl.W), np.int32)
        target = np.zeros((B, wl.W), np.int32)
    else:
        parents = np.empty((B, N), np.int32)
        draft = np.empty((B, N), np.int32)
        target = np.empty((B, N), np.int32)
        for b in range(B):
            if wl.tree == "worked":
                parents[b] = np.array([-1, 0, 0, 1, 2], np.int32)
            elif wl.tree == "random":
                parents[b] = random_tree(r_tree, N, wl.depth_cap)
            elif wl.tree == "eagle":
                parents[b] = eagle_tree(r_tree, wl.eagle_topk, wl.eagle_steps, N)
            elif wl.tree == "chain":
                parents[b] = chain_tree(N)
            else:
                raise ValueError(wl.tree)
            draft[b], target[b] = tokens_for(r_tok, parents[b],
                                             None if wl.tree == "worked" else 0.7)
    if prefix_lens is None:
        prefix_lens = np.full(B, wl.P, np.int32)
    prefix_lens = np.asarray(prefix_lens, np.int32)
    ps = wl.page_size
    max_pages = max(1, math.ceil((int(prefix_lens.max()) + wl.W) / ps))
    n_pages = 1 + B * max_pages
    page_table = (r_pt.permutation(n_pages - 1) + 1).astype(np.int32).reshape(B, max_pages)
    q = kc = vc = None
    if with_tensors:
        dt, kvt = TORCH_DTYPE[wl.dtype], TORCH_DTYPE[wl.kv]
        dev = torch.device(device)
        shape = (n_pages, wl.Hkv, ps, wl.D) if layout == "HND" else (n_pages, ps, wl.Hkv, wl.D)
        q = torch.empty((B, wl.R, wl.Hq, wl.D), dtype=dt, device=dev)
        kc = torch.empty(shape, dtype=kvt, device=dev)
        vc = torch.empty(shape, dtype=kvt, device=dev)
        for k, t in enumerate((q, kc, vc)):
            g = torch.Generator(device=dev)
            g.manual_seed(_torch_seed(seed, k))
            _randn_into(t, g)
        _poison(kc, vc, page_table, prefix_lens, wl, layout)
    return Inputs(wl, parents, draft, target, lm, prefix_lens, page_table, q, kc, vc, layout)


def _poison(kc, vc, page_table, prefix_lens, wl, layout):
    """NaN into page 0 and every slot past prefix + window."""
    nan = float("nan")
    kc[0] = nan
    vc[0] = nan
    ps = wl.page_size
    for b in range(page_table.shape[0]):
        end = int(prefix_lens[b]) + wl.W
        for lp in range(end // ps, page_table.shape[1]):
            first = max(0, end - lp * ps)
            if first >= ps:
                continue
            pg = int(page_table[b, lp])
            if layout == "HND":
                kc[pg, :, first:] = nan
                vc[pg, :, first:] = nan
            else:
                kc[pg, first:] = nan
                vc[pg, first:] = nan


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a bf16 (uint16 numpy) or FP8 E4M3 (uint8 numpy)
    tensor, or the fp32 values."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


# ---------------------------------------------------------------------------
# sampled verify inputs
# ---------------------------------------------------------------------------

SAMPLE_VOCAB = 128256   # vocabulary of the Llama-3 family (shapes only)


@dataclasses.dataclass
class SampleInputs:
    logits: torch.Tensor        # [B][N][V] (a view of [B][N][row_stride] when padded)
    temperature: np.ndarray     # [B] float32 (0 = greedy)
    seed: np.ndarray            # [B] uint64


def make_sample_inputs(B: int, N: int, V: int, seed: int, dtype: str = "bf16",
                       device="cpu", scale: float = 2.0, row_stride: Optional[int] = None,
                       temperatures=(0.0, 0.6, 1.0, 1.3)) -> SampleInputs:
    """Seeded target logits of every verify row, N(0, scale^2) drawn in fp32
    and rounded to the dtype, with a per-request temperature drawn from
    `temperatures` and a per-request 64-bit seed.  row_stride > V pads each
    row (the padding holds NaN, which no draw may read)."""
    r = _streams(seed + 104729, 1)[0]
    rs = V if row_stride is None else row_stride
    dev = torch.device(device)
    buf = torch.full((B, N, rs), float("nan"), dtype=TORCH_DTYPE[dtype], device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(_torch_seed(seed, 11))
    vals = torch.empty((B, N, V), dtype=TORCH_DTYPE[dtype], device=dev)
    _randn_into(vals, g)
    buf[:, :, :V] = vals * scale if dtype == "f32" else (vals.float() * scale).to(buf.dtype)
    temperature = r.choice(np.asarray(temperatures, np.float32), size=B).astype(np.float32)
    seeds = r.integers(0, 2 ** 63, size=B, dtype=np.int64).astype(np.uint64) * np.uint64(2) + \
        r.integers(0, 2, size=B).astype(np.uint64)
    return SampleInputs(buf[:, :, :V], temperature, seeds)


@dataclasses.dataclass
class RejectionInputs:
    probs: torch.Tensor          # float32 [B][N][V] (a view when the rows are padded)
    parents: np.ndarray          # int32 [B][N]
    draft: np.ndarray            # int32 [B][N]
    draft_score: np.ndarray      # float32 [B][N]
    coins: np.ndarray            # float32 [B][N], uniform in [0, 1)
    bonus_u: np.ndarray          # float32 [B][N], uniform in [0, 1)
    draft_q: Optional[torch.Tensor] = None   # float32 [B][N][V]: the drafter's rows


def make_rejection_inputs(B: int, N: int, V: int, seed: int, device="cpu", tree: str = "eagle",
                          scale: float = 2.0, row_stride: Optional[int] = None,
                          agree: float = 0.75, with_q: bool = False) -> RejectionInputs:
    """Seeded inputs of the sampled verify by rejection.  Trees: EAGLE top-8
    beam, random (depth <= 6) or a chain.  The target row after each node is
    a mix of softmax(N(0, scale^2)) and a point mass on a "hot" token of
    weight U(0.3, 0.9), in fp32.  A parent's first child drafts the hot token
    with probability `agree` and otherwise, like every later sibling, a
    token drawn from the parent's softmax part; a node's draft score is its
    parent's target probability of its token.  Coins and bonus draws are
    uniform fp32 in [0, 1).  row_stride > V pads the rows with NaN, which the
    walk never reads.  with_q adds the drafter's rows: the target's hot
    token at weight U(0.2, 0.8) over a softmax of fresh N(0, scale^2)
    logits, and then every child drafts a token drawn independently from its
    parent's q row (its draft score the q probability of that token)."""
    r = _streams(seed + 15485863, 1)[0]
    if tree == "eagle":
        parents = np.stack([eagle_tree(r, 8, 6, N) for _ in range(B)])
    elif tree == "chain":
        parents = np.tile(chain_tree(N), (B, 1))
    else:
        parents = np.stack([random_tree(r, N, 6) for _ in range(B)])
    parents = parents.astype(np.int32)
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(_torch_seed(seed, 13))
    rs = V if row_stride is None else row_stride
    buf = torch.full((B, N, rs), float("nan"), dtype=torch.float32, device=dev)
    logits = torch.empty((B, N, V), dtype=torch.float32, device=dev)
    _randn_into(logits, g)
    p0 = torch.softmax(logits * scale, -1)
    del logits
    hot = r.integers(0, V, (B, N))
    mix = r.uniform(0.3, 0.9, (B, N)).astype(np.float32)
    p = p0 * torch.as_tensor(1.0 - mix, device=dev)[..., None]
    p.view(B * N, V)[torch.arange(B * N, device=dev), torch.as_tensor(hot.reshape(-1), device=dev)] += \
        torch.as_tensor(mix.reshape(-1), device=dev)
    buf[:, :, :V] = p
    draws = torch.multinomial(p0.view(B * N, V), 8, replacement=True, generator=g)
    draws = draws.view(B, N, 8).cpu().numpy()
    del p0
    draft = np.zeros((B, N), np.int32)
    for b in range(B):
        seen = {}
        for c in range(1, N):
            n = int(parents[b, c])
            j = seen.get(n, 0)
            seen[n] = j + 1
            if j == 0 and r.random() < agree:
                draft[b, c] = hot[b, n]
            else:
                draft[b, c] = draws[b, n, j % 8]
    par_c = np.maximum(parents, 0)
    qv = None
    src = p
    if with_q:
        ql = torch.empty((B, N, V), dtype=torch.float32, device=dev)
        _randn_into(ql, g)
        qmix = r.uniform(0.2, 0.8, (B, N)).astype(np.float32)
        qv = torch.softmax(ql * scale, -1) * torch.as_tensor(1.0 - qmix, device=dev)[..., None]
        del ql
        qv.view(B * N, V)[torch.arange(B * N, device=dev),
                          torch.as_tensor(hot.reshape(-1), device=dev)] += \
            torch.as_tensor(qmix.reshape(-1), device=dev)
        qd = torch.multinomial(qv.view(B * N, V), 8, replacement=True, generator=g)
        qd = qd.view(B, N, 8).cpu().numpy()
        for b in range(B):
            seen = {}
            for c in range(1, N):
                n = int(parents[b, c])
                j = seen.get(n, 0)
                seen[n] = j + 1
                draft[b, c] = qd[b, n, j % 8]
        src = qv
    score = src[torch.as_tensor(np.arange(B)[:, None], device=dev),
                torch.as_tensor(par_c, device=dev), torch.as_tensor(draft.astype(np.int64), device=dev)]
    score = score.cpu().numpy().astype(np.float32)
    score[:, 0] = 1.0
    coins = r.random((B, N), dtype=np.float32)
    bonus_u = r.random((B, N), dtype=np.float32)
    if qv is not None:
        qbuf = torch.full((B, N, rs), float("nan"), dtype=torch.float32, device=dev)
        qbuf[:, :, :V] = qv
        qv = qbuf[:, :, :V]
    return RejectionInputs(buf[:, :, :V], parents, draft, score, coins, bonus_u, qv)


# ---------------------------------------------------------------------------
# MLA latent-cache inputs
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class MlaWorkload:
    name: str
    B: int
    P: int
    N: int
    Hq: int
    Dc: int          # kv_lora_rank: latent channels (scored against the query, and read as V)
    Dr: int          # rotary channels of the key
    page_size: int
    depth_cap: int = 6
    dtype: str = "bf16"
    kv_dtype: str = ""   # latent cache dtype when it differs from dtype: "fp8" (E4M3, bf16 q)

    @property
    def kv(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def W(self) -> int:
        return self.N

    @property
    def R(self) -> int:
        return self.N

    def with_(self, **kw) -> "MlaWorkload":
        return dataclasses.replace(self, **kw)

    def describe(self) -> str:
        dt = self.dtype if self.kv == self.dtype else "%s q, %s E4M3 latent cache" % (self.dtype,
                                                                                       self.kv)
        return ("%s: B %d, P %d, N %d random trees (depth <= %d), Hq %d, latent %d + rotary %d, "
                "%s, page size %d" % (self.name, self.B, self.P, self.N, self.depth_cap, self.Hq,
                                      self.Dc, self.Dr, dt, self.page_size))


MLA_WORKLOADS = {
    # one tensor-parallel share (16 of 128 heads) of a DeepSeek-style MLA layer
    "mla16": MlaWorkload("mla16", 8, 8192, 16, 16, 512, 64, 64),
    # every head of such a layer on one GPU
    "mla128": MlaWorkload("mla128", 4, 32768, 16, 128, 512, 64, 64),
    # the same two over an FP8 E4M3 latent cache
    "mla16_fp8": MlaWorkload("mla16_fp8", 8, 8192, 16, 16, 512, 64, 64, kv_dtype="fp8"),
    "mla128_fp8": MlaWorkload("mla128_fp8", 4, 32768, 16, 128, 512, 64, 64, kv_dtype="fp8"),
}


@dataclasses.dataclass
class MlaInputs:
    wl: MlaWorkload
    parents: np.ndarray          # [B][N]
    prefix_len: np.ndarray       # [B]
    page_table: np.ndarray       # [B][max_pages]
    q: torch.Tensor              # [B][N][Hq][Dc + Dr]
    latent: torch.Tensor         # [pages][page_size][Dc + Dr]

    @property
    def strides(self):
        """(page, token) strides in elements."""
        return (self.wl.page_size * (self.wl.Dc + self.wl.Dr), self.wl.Dc + self.wl.Dr)


def make_mla_inputs(wl: MlaWorkload, seed: int, device="cpu",
                    prefix_lens: Optional[np.ndarray] = None) -> MlaInputs:
    """Seeded MLA verify inputs: random trees, the absorbed query and the
    latent cache N(0, 1) (rounded to bf16, the latent cache to E4M3 under
    kv_dtype "fp8"), a shuffled page table; page 0 and every slot past
    prefix + window hold NaN."""
    r_tree, _, r_pt, _ = _streams(seed + 7777, 4)
    B, N = wl.B, wl.N
    parents = np.stack([random_tree(r_tree, N, wl.depth_cap) for _ in range(B)]).astype(np.int32)
    if prefix_lens is None:
        prefix_lens = np.full(B, wl.P, np.int32)
    prefix_lens = np.asarray(prefix_lens, np.int32)
    ps = wl.page_size
    max_pages = max(1, math.ceil((int(prefix_lens.max()) + wl.W) / ps))
    n_pages = 1 + B * max_pages
    page_table = (r_pt.permutation(n_pages - 1) + 1).astype(np.int32).reshape(B, max_pages)
    dt = TORCH_DTYPE[wl.dtype]
    dev = torch.device(device)
    Dk = wl.Dc + wl.Dr
    q = torch.empty((B, N, wl.Hq, Dk), dtype=dt, device=dev)
    lat = torch.empty((n_pages, ps, Dk), dtype=TORCH_DTYPE[wl.kv], device=dev)
    for k, t in enumerate((q, lat)):
        g = torch.Generator(device=dev)
        g.manual_seed(_torch_seed(seed + 7777, k))
        _randn_into(t, g)
    lat[0] = float("nan")
    for b in range(B):
        end = int(prefix_lens[b]) + wl.W
        for lp in range(end // ps, max_pages):
            first = max(0, end - lp * ps)
            if first < ps:
                lat[int(page_table[b, lp]), first:] = float("nan")
    return MlaInputs(wl, parents, prefix_lens, page_table, q, lat)
