"""GPU parity of tree construction (EAGLE-2 beam step, global selection with
pool-order or depth-first numbering, first-child / next-sibling links)
through the C ABI, against the CPU oracle.  Everything here is integer
output decided by fp32 comparisons that both sides make on the same fp32
values (the beam scores are single fp32 products), so every output is
compared bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verify_amd as tav
from tests.golden import load

pytestmark = pytest.mark.gpu


def say(*a):
    print("[build]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tav.lib()


def dev(x, dtype=torch.int32):
    return torch.as_tensor(np.ascontiguousarray(x)).to(dtype).cuda()


def host(t):
    return t.cpu().numpy()


def new_pool(B, C):
    return {"scores": np.zeros((B, C), np.float32), "parents": np.zeros((B, C), np.int32),
            "tokens": np.zeros((B, C), np.int32)}


@pytest.mark.parametrize("S,K", [(1, 8), (8, 8), (4, 16), (3, 5), (16, 64), (1, 1)])
def test_beam_step_bit_exact(S, K):
    rng = np.random.default_rng(S * 100 + K)
    B, base = 5, 7
    C = base + S * K + 3
    # scores and probabilities from a small set, so ties are common, plus NaN
    s = rng.choice([0.5, 0.25, 0.75, 1.0, np.nan], size=(B, S), p=[.3, .3, .2, .15, .05]).astype(np.float32)
    p = rng.choice([0.5, 0.125, 0.375, 0.25, np.nan], size=(B, S, K), p=[.3, .3, .2, .15, .05]).astype(np.float32)
    p[0] = rng.dirichlet(np.ones(K), size=S).astype(np.float32)
    idx = rng.integers(-1, base, size=(B, S)).astype(np.int32)
    tok = rng.integers(0, 32000, size=(B, S, K)).astype(np.int32)
    pool = new_pool(B, C)
    ns, ni = oracle.beam_step(s, idx, p, tok, pool, base)
    g = {k: dev(v, torch.float32 if k == "scores" else torch.int32) for k, v in new_pool(B, C).items()}
    gs, gi = tav.tree_beam_step(dev(s, torch.float32), dev(idx), dev(p, torch.float32), dev(tok),
                                g["scores"], g["parents"], g["tokens"], base)
    torch.cuda.synchronize()
    assert np.array_equal(host(g["scores"]).view(np.uint32), pool["scores"].view(np.uint32))
    assert np.array_equal(host(g["parents"]), pool["parents"])
    assert np.array_equal(host(g["tokens"]), pool["tokens"])
    assert np.array_equal(host(gs).view(np.uint32), ns.view(np.uint32))
    assert np.array_equal(host(gi), ni)


def test_beam_step_in_place():
    # the survivor arrays updated in place (n_surv == K)
    rng = np.random.default_rng(1)
    B, K, C = 4, 8, 8 + 64
    s = rng.random((B, K)).astype(np.float32)
    idx = np.tile(np.arange(K, dtype=np.int32), (B, 1))
    p = rng.dirichlet(np.ones(K), size=(B, K)).astype(np.float32)
    tok = rng.integers(0, 1000, size=(B, K, K)).astype(np.int32)
    pool = new_pool(B, C)
    ns, ni = oracle.beam_step(s, idx, p, tok, pool, K)
    gsc, gid = dev(s, torch.float32), dev(idx)
    g = {k: dev(v, torch.float32 if k == "scores" else torch.int32) for k, v in new_pool(B, C).items()}
    assert tav.lib().tree_beam_step(gsc.data_ptr(), gid.data_ptr(), dev(p, torch.float32).data_ptr(),
                                    dev(tok).data_ptr(), B, K, K, C, K, g["scores"].data_ptr(),
                                    g["parents"].data_ptr(), g["tokens"].data_ptr(),
                                    gsc.data_ptr(), gid.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert np.array_equal(host(gsc), ns) and np.array_equal(host(gid), ni)
    assert np.array_equal(host(g["parents"]), pool["parents"])


def eagle_pools(B, K, S, seed):
    """Per-step conditional probabilities (Dirichlet(1) per survivor slot)
    and tokens: drafter outputs, drawn up front."""
    rng = np.random.default_rng(seed)
    steps = []
    for i in range(S):
        n_s = 1 if i == 0 else K
        steps.append((rng.dirichlet(np.ones(K), size=(B, n_s)).astype(np.float32),
                      rng.integers(0, 128256, size=(B, n_s, K)).astype(np.int32)))
    return steps


@pytest.mark.parametrize("B,K,S,N", [(32, 8, 6, 64), (4, 4, 5, 8), (3, 2, 3, 5), (8, 10, 7, 64)])
def test_eagle_pipeline_bit_exact(B, K, S, N):
    """S beam steps, then the selection in both numberings and the links,
    on the GPU and in the oracle from the same drafter outputs; the
    selected trees then go through tree_build_masks."""
    C = K + (S - 1) * K * K
    steps = eagle_pools(B, K, S, B * 7 + K)
    pool = new_pool(B, C)
    s, idx = np.ones((B, 1), np.float32), np.full((B, 1), -1, np.int32)
    g = {k: dev(v, torch.float32 if k == "scores" else torch.int32) for k, v in new_pool(B, C).items()}
    gs, gi = dev(s, torch.float32), dev(idx)
    base = 0
    for p, tok in steps:
        s, idx = oracle.beam_step(s, idx, p, tok, pool, base)
        gs, gi = tav.tree_beam_step(gs, gi, dev(p, torch.float32), dev(tok), g["scores"],
                                    g["parents"], g["tokens"], base)
        base += p.shape[1] * K
    torch.cuda.synchronize()
    assert base == C
    assert np.array_equal(host(g["scores"]).view(np.uint32), pool["scores"].view(np.uint32))
    assert np.array_equal(host(g["parents"]), pool["parents"])
    roots = np.arange(B, dtype=np.int32) + 5
    for order in (0, 1):
        r = oracle.select_candidates(pool["scores"], pool["parents"], pool["tokens"], roots, N, order)
        gr = tav.tree_select_candidates(g["scores"], g["parents"], g["tokens"], dev(roots), N, order)
        torch.cuda.synchronize()
        for k in ("parents", "tokens", "selected", "tree_error"):
            assert np.array_equal(host(gr[k]), r[k]), (order, k)
        assert (r["tree_error"] == 0).all()
        nt, ns = oracle.retrieve_links(r["parents"])
        gnt, gns = tav.tree_retrieve_links(gr["parents"])
        m = tav.tree_build_masks(gr["parents"])
        torch.cuda.synchronize()
        assert np.array_equal(host(gnt), nt) and np.array_equal(host(gns), ns)
        rm = oracle.build_masks(r["parents"])
        assert np.array_equal(host(m["masks"]).view(np.uint64), rm["masks"])
        assert (host(m["tree_error"]) == 0).all()
    say("eagle pipeline B %d K %d S %d N %d: pool %d" % (B, K, S, N, C))


def random_pool(rng, C, bad=False, nan=False):
    pp = np.array([-1 if c == 0 or rng.random() < 0.2 else int(rng.integers(0, c))
                   for c in range(C)], np.int32)
    sc = np.empty(C, np.float32)
    for c in range(C):
        q = np.float32(rng.choice([1.0, 0.5, 0.75, 0.25, rng.random()]))
        sc[c] = q if pp[c] < 0 else sc[pp[c]] * q
    if nan:
        sc[rng.integers(0, C, size=max(1, C // 10))] = np.nan
    if bad:   # a child above its parent: the kept set may lose closure
        c = int(rng.integers(1, C))
        if pp[c] >= 0:
            sc[c] = sc[pp[c]] * 2 + 1
        else:
            pp[c] = c + 1 if c + 1 < C else -1   # a parent after its child
    return sc, pp


@pytest.mark.parametrize("C,N", [(328, 64), (68, 8), (8192, 64), (5, 6), (40, 1), (1000, 33),
                                 (63, 64)])
def test_select_random_pools_bit_exact(C, N):
    rng = np.random.default_rng(C + N)
    B = 12
    sc = np.empty((B, C), np.float32)
    pp = np.empty((B, C), np.int32)
    for b in range(B):
        sc[b], pp[b] = random_pool(rng, C, bad=(b % 4 == 3), nan=(b % 3 == 1))
    tk = rng.integers(0, 1000, size=(B, C)).astype(np.int32)
    roots = rng.integers(0, 1000, size=B).astype(np.int32)
    for order in (0, 1):
        r = oracle.select_candidates(sc, pp, tk, roots, N, order)
        gr = tav.tree_select_candidates(dev(sc, torch.float32), dev(pp), dev(tk), dev(roots), N, order)
        torch.cuda.synchronize()
        for k in ("parents", "tokens", "selected", "tree_error"):
            assert np.array_equal(host(gr[k]), r[k]), (C, N, order, k)
    say("C %d N %d: %d of %d requests rejected" % (C, N, int((r["tree_error"] > 0).sum()), B))


def test_retrieve_links_worked_and_random():
    gl = load("retrieve.txt")
    for k in ("eagle", "ddtree"):
        nt, ns = tav.tree_retrieve_links(dev(np.array([gl[k + "_parents"]])))
        torch.cuda.synchronize()
        assert host(nt)[0].tolist() == gl[k + "_next_token"]
        assert host(ns)[0].tolist() == gl[k + "_next_sibling"]
    rng = np.random.default_rng(4)
    for N in (1, 2, 17, 63, 64):
        par = np.array([[-1] + [int(rng.integers(0, i)) for i in range(1, N)] for _ in range(9)],
                       np.int32)
        nt, ns = oracle.retrieve_links(par)
        gnt, gns = tav.tree_retrieve_links(dev(par))
        torch.cuda.synchronize()
        assert np.array_equal(host(gnt), nt) and np.array_equal(host(gns), ns)
