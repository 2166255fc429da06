"""CPU fp64 oracle of the draft-tree verify path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding in ``tree_attention_verify_amd``) never imports, loads or calls
it, and the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over rows); this
module only builds it with gcc and marshals numpy arrays through ctypes.
Every function cites the page passage it follows in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc -O2 -fopenmp)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class OrcRows(ctypes.Structure):
    _fields_ = [
        ("base", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("prefix_len", ctypes.c_void_p),
        ("max_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("stride_page", ctypes.c_int64),
        ("stride_token", ctypes.c_int64),
        ("stride_head", ctypes.c_int64),
        ("stride_batch", ctypes.c_int64),
        ("n_heads", ctypes.c_int32),
        ("row_bytes", ctypes.c_int32),
    ]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.orc_build_masks.argtypes = [P, I, I, P, P, P, P, P]
        L.orc_shift_positions.argtypes = [P, P, I, I, I]
        L.orc_e4m3_decode.argtypes = [I]
        L.orc_e4m3_decode.restype = D
        L.orc_e4m3_round.argtypes = [D]
        L.orc_e4m3_round.restype = D
        L.orc_philox4x32_10.argtypes = [P, P, P]
        L.orc_philox4x32_10.restype = None
        L.orc_gumbel_uniform.argtypes = [ctypes.c_uint64, I64, I64]
        L.orc_gumbel_uniform.restype = D
        L.orc_sample_gumbel.argtypes = [P, I, I64, I, I, I, P, P, P, P, P, P]
        L.orc_sample_gumbel.restype = ctypes.c_int
        L.orc_beam_step.argtypes = [P, P, P, P, I, I, I, I, I, P, P, P, P, P]
        L.orc_beam_step.restype = ctypes.c_int
        L.orc_select_candidates.argtypes = [P, P, P, P, I, I, I, I, P, P, P, P]
        L.orc_select_candidates.restype = ctypes.c_int
        L.orc_retrieve_links.argtypes = [P, I, I, P, P]
        L.orc_retrieve_links.restype = ctypes.c_int
        L.orc_mla_attention.argtypes = [P, P, I, I, I64, I64, P, I, I, P, P, I, I, I, I, I, I,
                                        D, P, I64, P, P]
        L.orc_mla_attention.restype = ctypes.c_int
        L.orc_tree_attention.argtypes = [P, P, P, I, I, I64, I64, I64, P, I, I, P, I,
                                         P, I, I, I, I, I, I, D, P, I64, P, P]
        L.orc_causal_attention.argtypes = [P, P, P, I, I, I, I, I, I, D, P, P]
        L.orc_merge.argtypes = [P, P, I, I, I, P, P]
        L.orc_verify_greedy.argtypes = [P, P, P, I, I, P, P, P]
        L.orc_verify_rejection.argtypes = [P, I64, I, P, P, P, P, P, I, I, P, P, P, P]
        L.orc_verify_rejection.restype = ctypes.c_int
        L.orc_verify_rejection_q.argtypes = [P, I64, P, I64, I, P, P, P, P, P, I, I, P, P, P, P]
        L.orc_verify_rejection_q.restype = ctypes.c_int
        L.orc_compact_rows.argtypes = [ctypes.POINTER(OrcRows), I, P, P, I, I]
        for f in ("orc_build_masks", "orc_shift_positions", "orc_tree_attention",
                  "orc_causal_attention", "orc_merge", "orc_verify_greedy",
                  "orc_compact_rows"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:  # raw bf16 bit patterns
        return 1
    if a.dtype == np.uint8:   # raw FP8 E4M3 codes (K/V caches only)
        return 2
    raise TypeError("oracle inputs are float32, raw bf16 (uint16) or raw E4M3 (uint8) arrays, "
                    "got %s" % a.dtype)


def e4m3_decode(codes) -> np.ndarray:
    """fp64 values of FP8 E4M3 codes (the oracle's decoder)."""
    codes = np.asarray(codes, dtype=np.int64).ravel()
    return np.array([lib().orc_e4m3_decode(int(c)) for c in codes], np.float64)


def e4m3_round(x) -> np.ndarray:
    """Each value rounded to the nearest E4M3 value (ties to even, saturating
    at +-448, NaN kept), as fp64."""
    x = np.asarray(x, np.float64).ravel()
    return np.array([lib().orc_e4m3_round(float(v)) for v in x], np.float64)


def _check(rc, name):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments" % name)


def build_masks(parents, vc=None):
    """parents int32 [B][N] -> dict(depth, masks uint64, positions, tree_error)."""
    parents = _c(parents, np.int32)
    B, N = parents.shape
    depth = np.empty((B, N), np.int32)
    masks = np.empty((B, N), np.uint64)
    err = np.empty((B,), np.int32)
    pos = None
    if vc is not None:
        vc = _c(vc, np.int32)
        pos = np.empty((B, N), np.int32)
    _check(lib().orc_build_masks(_p(parents), B, N, _p(vc), _p(depth), _p(masks),
                                 _p(pos), _p(err)), "build_masks")
    return {"depth": depth, "masks": masks, "positions": pos, "tree_error": err}


def shift_positions(pos, depth, direction):
    pos = np.array(pos, dtype=np.int32, copy=True, order="C")
    depth = _c(depth, np.int32)
    B, N = pos.shape
    _check(lib().orc_shift_positions(_p(pos), _p(depth), B, N, int(direction)),
           "shift_positions")
    return pos


def tree_attention(q, k_cache, v_cache, strides, page_table, page_size, prefix_len,
                   masks, W, Hkv, prefix_window=0, sm_scale=0.0, rows=None):
    """fp64 tree attention.

    q: [B][R][Hq][D] float32 or uint16 (bf16 bits); k_cache/v_cache: flat pools
    of the same dtype addressed with ``strides`` = (page, head, token) in
    elements; page_table int32 [B][max_pages]; prefix_len int32 [B];
    masks uint64 [B][R].  Returns (out float64, lse2 float64) of shape
    [B][R][Hq][D] / [B][R][Hq], or [n][D] / [n] for a ``rows`` list of flat
    row ids ((b*R + r)*Hq + h).
    """
    q = np.ascontiguousarray(q)
    dt = _dtype_code(q)
    k_cache = np.ascontiguousarray(k_cache)
    v_cache = np.ascontiguousarray(v_cache)
    kvdt = _dtype_code(k_cache)
    assert v_cache.dtype == k_cache.dtype
    assert kvdt == dt or (kvdt == 2 and dt == 1), "FP8 caches take a bf16 query"
    assert dt != 2, "the query is fp32 or bf16"
    B, R, Hq, D = q.shape
    page_table = _c(page_table, np.int32)
    prefix_len = _c(prefix_len, np.int32)
    masks = _c(masks, np.uint64)
    assert masks.shape == (B, R)
    if rows is None:
        out = np.empty((B, R, Hq, D), np.float64)
        lse = np.empty((B, R, Hq), np.float64)
        rp, nr = None, 0
    else:
        rows = _c(rows, np.int64)
        out = np.empty((rows.size, D), np.float64)
        lse = np.empty((rows.size,), np.float64)
        rp, nr = rows, rows.size
    sp, sh, st = (int(x) for x in strides)
    _check(lib().orc_tree_attention(
        _p(q), _p(k_cache), _p(v_cache), dt, kvdt, sp, sh, st, _p(page_table),
        page_table.shape[1], int(page_size), _p(prefix_len), int(prefix_window),
        _p(masks), int(W), B, R, Hq, int(Hkv), D, float(sm_scale), _p(rp), nr,
        _p(out), _p(lse)), "tree_attention")
    return out, lse


def causal_attention(q, k, v, sm_scale=0.0):
    """q [n][Hq][D], k/v [L][Hkv][D] (float32 or bf16 bits) -> fp64 (out, lse2)."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    dt = _dtype_code(q)
    n, Hq, D = q.shape
    L, Hkv, _ = k.shape
    out = np.empty((n, Hq, D), np.float64)
    lse = np.empty((n, Hq), np.float64)
    _check(lib().orc_causal_attention(_p(q), _p(k), _p(v), dt, n, L, Hq, Hkv, D,
                                      float(sm_scale), _p(out), _p(lse)), "causal")
    return out, lse


def merge(o_parts, lse2_parts):
    """o_parts [S][n][D], lse2_parts [S][n] (float64) -> merged (out, lse2)."""
    o_parts = _c(o_parts, np.float64)
    lse2_parts = _c(lse2_parts, np.float64)
    S, n, D = o_parts.shape
    out = np.empty((n, D), np.float64)
    lse = np.empty((n,), np.float64)
    _check(lib().orc_merge(_p(o_parts), _p(lse2_parts), S, n, D, _p(out), _p(lse)),
           "merge")
    return out, lse


def verify_greedy(draft, target, parents):
    draft = _c(draft, np.int32)
    target = _c(target, np.int32)
    parents = _c(parents, np.int32)
    B, N = parents.shape
    path = np.empty((B, N), np.int32)
    alen = np.empty((B,), np.int32)
    tok = np.empty((B, N), np.int32)
    _check(lib().orc_verify_greedy(_p(draft), _p(target), _p(parents), B, N,
                                   _p(path), _p(alen), _p(tok)), "verify_greedy")
    return {"accepted_path": path, "accept_len": alen, "accepted_tokens": tok}


def verify_rejection(probs, draft, parents, coins, bonus_u, draft_score=None):
    """Tree rejection sampling ([DDT] "The Implementation"; [DTS] "Sampled
    verify keys noise by position"): probs float32 [B][N][V] target weights
    per node, draft / parents int32 [B][N], coins / bonus_u float32 [B][N]
    uniform in [0, 1), draft_score float32 [B][N] or None.  Returns the path,
    accept_len, emitted tokens and, per request, how near its children's
    tests came to a tie (relative margin)."""
    probs = _c(probs, np.float32)
    draft = _c(draft, np.int32)
    parents = _c(parents, np.int32)
    coins = _c(coins, np.float32)
    bonus_u = _c(bonus_u, np.float32)
    B, N, V = probs.shape
    sc = None if draft_score is None else _c(draft_score, np.float32)
    path = np.empty((B, N), np.int32)
    alen = np.empty((B,), np.int32)
    tok = np.empty((B, N), np.int32)
    margin = np.empty((B,), np.float64)
    _check(lib().orc_verify_rejection(_p(probs), V, V, _p(draft), _p(parents),
                                      None if sc is None else _p(sc), _p(coins), _p(bonus_u),
                                      B, N, _p(path), _p(alen), _p(tok), _p(margin)),
           "verify_rejection")
    return {"accepted_path": path, "accept_len": alen, "accepted_tokens": tok, "margin": margin}


def verify_rejection_q(probs, draft_q, draft, parents, coins, bonus_u, draft_score=None):
    """Tree rejection sampling against the draft distribution of each node's
    children ([DTS] "Sampled verify keys noise by position"): draft_q
    float32 [B][N][V], row n the distribution that drew node n's children;
    the rest as verify_rejection."""
    probs = _c(probs, np.float32)
    draft_q = _c(draft_q, np.float32)
    draft = _c(draft, np.int32)
    parents = _c(parents, np.int32)
    coins = _c(coins, np.float32)
    bonus_u = _c(bonus_u, np.float32)
    B, N, V = probs.shape
    assert draft_q.shape == (B, N, V)
    sc = None if draft_score is None else _c(draft_score, np.float32)
    path = np.empty((B, N), np.int32)
    alen = np.empty((B,), np.int32)
    tok = np.empty((B, N), np.int32)
    margin = np.empty((B,), np.float64)
    _check(lib().orc_verify_rejection_q(_p(probs), V, _p(draft_q), V, V, _p(draft), _p(parents),
                                        None if sc is None else _p(sc), _p(coins), _p(bonus_u),
                                        B, N, _p(path), _p(alen), _p(tok), _p(margin)),
           "verify_rejection_q")
    return {"accepted_path": path, "accept_len": alen, "accepted_tokens": tok, "margin": margin}


def compact_rows(tables, accepted_path, accept_len):
    """In-place compaction of host buffers.

    tables: list of dicts with keys buf (writable numpy array, any dtype),
    page_table (int32 [B][max_pages] or None), prefix_len (int32 [B] or None),
    page_size, stride_page, stride_token, stride_head, stride_batch (bytes),
    n_heads, row_bytes.
    """
    accepted_path = _c(accepted_path, np.int32)
    accept_len = _c(accept_len, np.int32)
    B, N = accepted_path.shape
    arr = (OrcRows * len(tables))()
    keep = []
    for i, t in enumerate(tables):
        buf = t["buf"]
        assert buf.flags.c_contiguous and buf.flags.writeable
        pt = t.get("page_table")
        pl = t.get("prefix_len")
        if pt is not None:
            pt = _c(pt, np.int32)
            pl = _c(pl, np.int32)
            keep += [pt, pl]
        arr[i] = OrcRows(buf.ctypes.data, _p(pt), _p(pl),
                         0 if pt is None else pt.shape[1], int(t.get("page_size", 1)),
                         int(t.get("stride_page", 0)), int(t["stride_token"]),
                         int(t.get("stride_head", 0)), int(t.get("stride_batch", 0)),
                         int(t.get("n_heads", 1)), int(t["row_bytes"]))
    _check(lib().orc_compact_rows(arr, len(tables), _p(accepted_path), _p(accept_len),
                                  B, N), "compact_rows")


def philox4x32_10(ctr, key) -> np.ndarray:
    """Philox4x32-10 of one 4-word counter under a 2-word key (uint32)."""
    c = _c(np.asarray(ctr, np.uint32), np.uint32)
    k = _c(np.asarray(key, np.uint32), np.uint32)
    out = np.empty(4, np.uint32)
    lib().orc_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def gumbel_uniform(seed, pos, v) -> float:
    """The uniform in (0, 1) of token v at key position pos under seed."""
    return float(lib().orc_gumbel_uniform(int(seed) & (2**64 - 1), int(pos), int(v)))


def sample_gumbel(logits, temperature, seed, positions):
    """Gumbel-max sampled target token of every verify row.

    logits: [B][N][V] float32 or uint16 (bf16 bits); temperature float [B]
    (<= 0: greedy); seed uint64 [B]; positions int32 [B][N] (vc + depth, the
    node's own position: the key is the position it predicts, one more).
    Returns (tokens int32 [B][N], zmax float64 [B][N], z2 float64 [B][N]):
    the winning perturbed score and the best score of any other token.
    """
    logits = np.ascontiguousarray(logits)
    dt = _dtype_code(logits)
    assert dt in (0, 1)
    B, N, V = logits.shape
    temperature = _c(temperature, np.float32)
    seed = _c(np.asarray(seed, np.uint64), np.uint64)
    positions = _c(positions, np.int32)
    assert temperature.shape == (B,) and seed.shape == (B,) and positions.shape == (B, N)
    tokens = np.empty((B, N), np.int32)
    zmax = np.empty((B, N), np.float64)
    z2 = np.empty((B, N), np.float64)
    _check(lib().orc_sample_gumbel(_p(logits), dt, V, V, B, N, _p(temperature), _p(seed),
                                   _p(positions), _p(tokens), _p(zmax), _p(z2)), "sample_gumbel")
    return tokens, zmax, z2


def beam_step(scores, surv_idx, child_p, child_tok, pool, pool_base):
    """One EAGLE-2 expansion step.  scores float32 [B][S], surv_idx int32
    [B][S], child_p float32 [B][S][K], child_tok int32 [B][S][K]; pool = dict
    of "scores" float32 [B][C], "parents" int32 [B][C], "tokens" int32 [B][C],
    updated in place at entries pool_base .. pool_base + S*K - 1.  Returns
    (next_scores float32 [B][K], next_idx int32 [B][K])."""
    scores = _c(scores, np.float32)
    surv_idx = _c(surv_idx, np.int32)
    child_p = _c(child_p, np.float32)
    child_tok = _c(child_tok, np.int32)
    B, S, K = child_p.shape
    C = pool["scores"].shape[1]
    for k in ("scores", "parents", "tokens"):
        assert pool[k].flags.c_contiguous
    ns = np.empty((B, K), np.float32)
    ni = np.empty((B, K), np.int32)
    _check(lib().orc_beam_step(_p(scores), _p(surv_idx), _p(child_p), _p(child_tok), B, S, K, C,
                               int(pool_base), _p(pool["scores"]), _p(pool["parents"]),
                               _p(pool["tokens"]), _p(ns), _p(ni)), "beam_step")
    return ns, ni


def select_candidates(pool_scores, pool_parents, pool_tokens, root_tokens, N, order=0):
    """The verify tree from a candidate pool: the N - 1 best candidates
    (score descending, lower pool index on ties, NaN last), numbered by pool
    order (order 0) or depth first best child first (order 1), the root as
    node 0.  Returns dict(parents, tokens, selected int32 [B][N],
    tree_error int32 [B])."""
    sc = _c(pool_scores, np.float32)
    pp = _c(pool_parents, np.int32)
    pt = _c(pool_tokens, np.int32)
    rt = _c(root_tokens, np.int32)
    B, C = sc.shape
    out = {k: np.empty((B, N), np.int32) for k in ("parents", "tokens", "selected")}
    out["tree_error"] = np.empty((B,), np.int32)
    _check(lib().orc_select_candidates(_p(sc), _p(pp), _p(pt), _p(rt), B, C, int(N), int(order),
                                       _p(out["parents"]), _p(out["tokens"]),
                                       _p(out["selected"]), _p(out["tree_error"])),
           "select_candidates")
    return out


def retrieve_links(parents):
    """(next_token, next_sibling) int32 [B][N]: first child and next sibling
    in node order, -1 where there is none."""
    par = _c(parents, np.int32)
    B, N = par.shape
    nt = np.empty((B, N), np.int32)
    nsb = np.empty((B, N), np.int32)
    _check(lib().orc_retrieve_links(_p(par), B, N, _p(nt), _p(nsb)), "retrieve_links")
    return nt, nsb


def mla_attention(q, latent, strides, page_table, page_size, prefix_len, masks, W, Dc, Dr,
                  sm_scale=0.0, rows=None):
    """fp64 tree attention over an MLA latent cache.

    q: [B][R][Hq][Dc + Dr] float32 or uint16 (bf16 bits); latent: a flat
    pool of the same dtype, or of uint8 E4M3 codes under a bf16 query (every
    key is then scored with the query rounded to E4M3), with (page, token)
    strides in elements, Dc + Dr contiguous channels per token (latent part,
    then rotary part).  Returns (out float64 [B][R][Hq][Dc], lse2 float64
    [B][R][Hq]) or, for a rows list, ([n][Dc], [n])."""
    q = np.ascontiguousarray(q)
    dt = _dtype_code(q)
    latent = np.ascontiguousarray(latent)
    ldt = _dtype_code(latent)
    assert dt in (0, 1) and (ldt == dt or (ldt == 2 and dt == 1)), \
        "the latent pool is the query's dtype, or E4M3 under a bf16 query"
    B, R, Hq, Dk = q.shape
    assert Dk == Dc + Dr
    page_table = _c(page_table, np.int32)
    prefix_len = _c(prefix_len, np.int32)
    masks = _c(masks, np.uint64)
    if rows is None:
        out = np.empty((B, R, Hq, Dc), np.float64)
        lse = np.empty((B, R, Hq), np.float64)
        rp, nr = None, 0
    else:
        rows = _c(rows, np.int64)
        out = np.empty((rows.size, Dc), np.float64)
        lse = np.empty((rows.size,), np.float64)
        rp, nr = rows, rows.size
    sp, st = (int(x) for x in strides)
    _check(lib().orc_mla_attention(_p(q), _p(latent), dt, ldt, sp, st, _p(page_table),
                                   page_table.shape[1], int(page_size), _p(prefix_len),
                                   _p(masks), int(W), B, R, Hq, int(Dc), int(Dr),
                                   float(sm_scale), _p(rp), nr, _p(out), _p(lse)),
           "mla_attention")
    return out, lse
