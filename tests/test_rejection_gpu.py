"""GPU parity of the sampled verify by tree rejection sampling through the C
ABI, against the CPU fp64 oracle.

Every decision of the walk compares fp32 sums in the kernel and fp64 sums
in the oracle.  The path and the drafted tokens must match the oracle's,
unless the oracle reports that one of the children's tests came within
MARGIN (relative to the row total) of a tie, and at most MAX_WALKS_OFF
requests per case may differ that way.
The bonus token is a draw by inverse CDF, where a single token can hold
less of the row than the fp32 error of a running sum over 128256 tokens, so
it must match the oracle's or be a token whose fp64 running-sum interval
(of the residual row at the last node) holds the draw's target within
CDF_TOL of the row's residual total, for at most MAX_BONUS_OFF requests per
case.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verify_amd as tav
from tree_attention_verify_amd import inputs as gen

pytestmark = pytest.mark.gpu

MARGIN = 2e-5
CDF_TOL = 2e-5
# Bounds on the differences per case, set just above what the seeded cases
# show (every walk equal, at most one bonus draw resolved differently by
# fp32 rounding): a walk may differ only at a near tie, and at most one per
# case; at most two bonus draws per case may differ, each within CDF_TOL.
MAX_WALKS_OFF = 1
MAX_BONUS_OFF = 2


def say(*a):
    print("[rejection]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tav.lib()


def dev(x, dtype=torch.int32):
    return torch.as_tensor(np.ascontiguousarray(x)).to(dtype).cuda()


def run_and_check(x, with_score=True, tag="", max_near=None):
    B, N, V = x.probs.shape
    probs = x.probs if x.probs.is_cuda else x.probs.cuda()
    score = dev(x.draft_score, torch.float32) if with_score else None
    r = tav.verify_tree_rejection(probs, dev(x.draft), dev(x.parents), dev(x.coins, torch.float32),
                                  dev(x.bonus_u, torch.float32), draft_score=score)
    torch.cuda.synchronize()
    ref = oracle.verify_rejection(np.ascontiguousarray(x.probs.cpu().numpy()), x.draft, x.parents,
                                  x.coins, x.bonus_u, x.draft_score if with_score else None)
    path = r["accepted_path"].cpu().numpy()
    alen = r["accept_len"].cpu().numpy()
    tok = r["accepted_tokens"].cpu().numpy()
    walk_same = (path == ref["accepted_path"]).all(1) & (alen == ref["accept_len"])
    near = ref["margin"] < MARGIN
    bad = np.nonzero(~walk_same & ~near)[0]
    assert bad.size == 0, (tag, bad[:5], path[bad[:1]], ref["accepted_path"][bad[:1]])
    assert (~walk_same).sum() <= (max_near if max_near is not None else MAX_WALKS_OFF), tag
    probs_h = None
    n_cdf = 0
    for b in np.nonzero(walk_same)[0]:
        L = int(alen[b])
        assert (tok[b, :L - 1] == ref["accepted_tokens"][b, :L - 1]).all()
        assert (tok[b, L:] == -1).all()
        if tok[b, L - 1] == ref["accepted_tokens"][b, L - 1]:
            continue
        # the bonus: the residual at the last node (its children's tokens
        # removed, unless the path is full) by numpy's fp64 cumulative sum
        if probs_h is None:
            probs_h = x.probs.cpu().numpy()
        cur = int(path[b, L - 1])
        row = probs_h[b, cur].astype(np.float64)
        r = np.where(np.isfinite(row) & (row > 0), row, 0.0)
        if L < N:
            for c in np.nonzero(x.parents[b] == cur)[0]:
                if 0 <= x.draft[b, c] < V:
                    r[x.draft[b, c]] = 0.0
        c = np.cumsum(r)
        target = float(x.bonus_u[b, cur]) * c[-1]
        g = int(tok[b, L - 1])
        assert 0 <= g < V and r[g] > 0, (tag, b, g)
        assert c[g] - r[g] <= target + CDF_TOL * c[-1] and c[g] >= target - CDF_TOL * c[-1], \
            (tag, b, g, int(ref["accepted_tokens"][b, L - 1]), c[g] - r[g], target, c[g])
        n_cdf += 1
    say(tag, "B %d N %d V %d: %d of %d walks equal (%d near a tie), %d bonus draws off by "
        "rounding, mean accept_len %.2f" % (B, N, V, int(walk_same.sum()), B, int(near.sum()),
                                            n_cdf, float(alen.mean())))
    assert n_cdf <= MAX_BONUS_OFF, tag
    # the walk is a path from the root through parent links
    for b in range(B):
        p = path[b, :alen[b]]
        assert p[0] == 0 and all(x.parents[b, p[k + 1]] == p[k] for k in range(len(p) - 1))
    return alen


CASES = {
    # name: (B, N, V, tree, row_stride, agree)
    "eagle_tiles": (64, 64, 3000, "eagle", None, 0.75),
    "random_ragged": (128, 16, 1000, "random", None, 0.9),
    "chain_deep": (64, 16, 2048, "chain", None, 1.0),
    "one_tile": (64, 8, 257, "random", 260, 0.9),
    "tiny_vocab": (64, 8, 3, "random", 4, 0.9),
    "padded_rows": (32, 32, 1000, "random", 1004, 0.9),
    "single_node": (16, 1, 500, "chain", None, 1.0),
    # several workgroups per request: 782 tiles in 13 slices (the last one
    # partial, its last tile 64 tokens), 13 workgroups per request
    "many_slices": (2, 64, 200000, "eagle", None, 0.75),
    # the largest vocabulary: 64 slices, 64 workgroups per request
    "max_vocab": (2, 16, 1 << 20, "random", None, 0.9),
    # 5 slices over 3 workgroups per request (members take 2, 2 and 1)
    "uneven_slices": (100, 16, 70000, "eagle", None, 0.75),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_rejection_parity(name):
    B, N, V, tree, rs, agree = CASES[name]
    say("case", name)
    x = gen.make_rejection_inputs(B, N, V, 31, "cuda", tree=tree, row_stride=rs, agree=agree)
    alen = run_and_check(x, tag=name)
    if name == "chain_deep":
        assert alen.max() >= 5


def test_rejection_index_order_without_scores():
    x = gen.make_rejection_inputs(64, 64, 2000, 32, "cuda", tree="eagle", agree=0.9)
    run_and_check(x, with_score=False, tag="no scores")


def test_rejection_special_values():
    """NaN, infinite and negative target entries carry no weight; draft
    tokens outside [0, V) are rejected; an all-zero row's bonus is token 0;
    coins of 0 accept the best-scored child with weight."""
    B, N, V = 8, 16, 700
    x = gen.make_rejection_inputs(B, N, V, 33, "cpu", tree="random", agree=1.0)
    p = x.probs.clone()
    p[0, 0, :50] = float("nan")
    p[1, 0, 100:200] = float("inf")
    p[2, 0, :] = -1.0
    p[2, 0, 3] = 0.5
    p[3] = 0.0
    x.draft[4, 1:] = -1
    x.draft[5, 1:4] = V + 7
    x.coins[6] = 0.0
    x.bonus_u[7] = np.nextafter(np.float32(1), np.float32(0))
    x = gen.RejectionInputs(p.cuda(), x.parents, x.draft, x.draft_score, x.coins, x.bonus_u)
    run_and_check(x, tag="special values", max_near=1)


def test_rejection_full_size_every_request():
    """The benchmark's shape: 32 requests x 64 rows (EAGLE top-8 trees), a
    128256-token vocabulary; every request against the oracle."""
    x = gen.make_rejection_inputs(32, 64, gen.SAMPLE_VOCAB, 4, "cuda", tree="eagle")
    run_and_check(x, tag="full size")


def test_rejection_emits_the_target_law_on_gpu():
    """20000 walks of one small tree: the first emitted token follows the
    root's target row (chi-square, 4 dof), as in the oracle's pin."""
    rng = np.random.default_rng(17)
    V, N, B = 5, 6, 20000
    par = np.array([-1, 0, 0, 0, 1, 1], np.int32)
    draft = np.array([0, 2, 0, 4, 1, 3], np.int32)
    score = np.array([0.0, 0.2, 0.5, 0.3, 0.6, 0.1], np.float32)
    rows = (rng.dirichlet(np.ones(V), N) * rng.uniform(0.5, 3.0, (N, 1))).astype(np.float32)
    buf = torch.full((B, N, 8), float("nan"), dtype=torch.float32)   # rows padded to 8
    buf[:, :, :V] = torch.as_tensor(rows)
    probs = buf.cuda()[:, :, :V]
    r = tav.verify_tree_rejection(probs, dev(np.tile(draft, (B, 1))), dev(np.tile(par, (B, 1))),
                                  dev(rng.random((B, N), np.float32), torch.float32),
                                  dev(rng.random((B, N), np.float32), torch.float32),
                                  draft_score=dev(np.tile(score, (B, 1)), torch.float32))
    t1 = r["accepted_tokens"][:, 0].cpu().numpy()
    cnt = np.bincount(t1, minlength=V)
    exp = rows[0].astype(np.float64) / rows[0].astype(np.float64).sum() * B
    assert float(((cnt - exp) ** 2 / exp).sum()) < 20.5


def _residual_q(p_row, q_row, n_rejected):
    """fp64 residual after n rejections against q (for the bonus bracket)."""
    w = np.where(np.isfinite(p_row) & (p_row > 0), p_row, 0).astype(np.float64)
    qw = np.where(np.isfinite(q_row) & (q_row > 0), q_row, 0).astype(np.float64)
    r = w / w.sum() if w.sum() > 0 else w
    qh = qw / qw.sum() if qw.sum() > 0 else qw
    for _ in range(n_rejected):
        r = np.maximum(r - qh, 0.0)
        z = r.sum()
        r = r / z if z > 0 else r * 0.0
    return r


def run_and_check_q(x, tag=""):
    B, N, V = x.probs.shape
    r = tav.verify_tree_rejection(x.probs, dev(x.draft), dev(x.parents), dev(x.coins, torch.float32),
                                  dev(x.bonus_u, torch.float32),
                                  draft_score=dev(x.draft_score, torch.float32), draft_q=x.draft_q)
    torch.cuda.synchronize()
    ph = np.ascontiguousarray(x.probs.cpu().numpy())
    qh = np.ascontiguousarray(x.draft_q.cpu().numpy())
    ref = oracle.verify_rejection_q(ph, qh, x.draft, x.parents, x.coins, x.bonus_u, x.draft_score)
    path = r["accepted_path"].cpu().numpy()
    alen = r["accept_len"].cpu().numpy()
    tok = r["accepted_tokens"].cpu().numpy()
    walk_same = (path == ref["accepted_path"]).all(1) & (alen == ref["accept_len"])
    near = ref["margin"] < MARGIN
    bad = np.nonzero(~walk_same & ~near)[0]
    assert bad.size == 0, (tag, bad[:5], path[bad[:1]], ref["accepted_path"][bad[:1]])
    assert (~walk_same).sum() <= MAX_WALKS_OFF, tag
    n_cdf = 0
    for b in np.nonzero(walk_same)[0]:
        L = int(alen[b])
        assert (tok[b, :L - 1] == ref["accepted_tokens"][b, :L - 1]).all()
        if tok[b, L - 1] == ref["accepted_tokens"][b, L - 1]:
            continue
        cur = int(path[b, L - 1])
        nrej = int((x.parents[b] == cur).sum()) if L < N else 0
        res = _residual_q(ph[b, cur], qh[b, cur], nrej)
        c = np.cumsum(res)
        target = float(x.bonus_u[b, cur]) * c[-1]
        g = int(tok[b, L - 1])
        assert res[g] > 0 and c[g] - res[g] <= target + CDF_TOL * c[-1] \
            and c[g] >= target - CDF_TOL * c[-1], (tag, b, g)
        n_cdf += 1
    say(tag, "q form, B %d N %d V %d: %d of %d walks equal (%d near a tie), %d bonus draws off by "
        "rounding, mean accept_len %.2f" % (B, N, V, int(walk_same.sum()), B, int(near.sum()),
                                            n_cdf, float(alen.mean())))
    assert n_cdf <= MAX_BONUS_OFF, tag


@pytest.mark.parametrize("name", ["eagle_tiles", "random_ragged", "chain_deep", "padded_rows",
                                  "one_tile", "many_slices", "max_vocab"])
def test_rejection_against_q_parity(name):
    B, N, V, tree, rs, agree = CASES[name]
    x = gen.make_rejection_inputs(B, N, V, 41, "cuda", tree=tree, row_stride=rs, agree=agree,
                                  with_q=True)
    run_and_check_q(x, tag="q " + name)


def test_rejection_against_q_full_size():
    x = gen.make_rejection_inputs(32, 64, gen.SAMPLE_VOCAB, 4, "cuda", tree="eagle", with_q=True)
    run_and_check_q(x, tag="q full size")


@pytest.mark.parametrize("form", ["fixed", "q"])
def test_rejection_full_path_on_a_64_node_chain(form):
    """Every target row puts all its weight on the next node's drafted
    token: the walk takes all 64 nodes and the bonus is drawn at node 63 with
    nothing rejected there (against q too, with q equal to the target)."""
    B, N, V = 16, 64, 1000
    rng = np.random.default_rng(51)
    par = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    draft = rng.integers(0, V, (B, N)).astype(np.int32)
    p = np.zeros((B, N, V), np.float32)
    for n in range(N - 1):
        p[np.arange(B), n, draft[:, n + 1]] = 1.0
    p[:, N - 1, :] = rng.random((B, V)).astype(np.float32)
    coins = rng.random((B, N)).astype(np.float32)
    bu = rng.random((B, N)).astype(np.float32)
    pt = torch.as_tensor(p).cuda()
    r = tav.verify_tree_rejection(pt, dev(draft), dev(par), dev(coins, torch.float32),
                                  dev(bu, torch.float32), draft_q=pt if form == "q" else None)
    if form == "q":
        ref = oracle.verify_rejection_q(p, p, draft, par, coins, bu)
    else:
        ref = oracle.verify_rejection(p, draft, par, coins, bu)
    alen = r["accept_len"].cpu().numpy()
    assert (alen == N).all() and (ref["accept_len"] == N).all()
    assert np.array_equal(r["accepted_path"].cpu().numpy(), ref["accepted_path"])
    tok = r["accepted_tokens"].cpu().numpy()
    assert np.array_equal(tok[:, :N - 1], ref["accepted_tokens"][:, :N - 1])
    c = np.cumsum(p[:, N - 1].astype(np.float64), 1)
    for b in range(B):       # the bonus: the inverse CDF of node 63's row
        g = int(tok[b, N - 1])
        target = float(bu[b, N - 1]) * c[b, -1]
        lo = c[b, g] - float(p[b, N - 1, g])
        assert lo <= target + CDF_TOL * c[b, -1] and c[b, g] >= target - CDF_TOL * c[b, -1]


def test_rejection_workspace_reused_across_calls():
    """One workspace serves calls of different shapes and both forms in a
    row (each call clears the counters it uses): every result is bit-identical
    to a call with a fresh workspace, and to a repeat of itself."""
    big = tav.verify_tree_rejection_workspace_size(32, 64, 70000)
    ws = torch.full((big,), 0xA5, dtype=torch.uint8, device="cuda")   # not zero to begin with
    for B, N, V, seed, with_q in [(32, 64, 70000, 61, False), (8, 16, 3000, 62, True),
                                  (32, 64, 70000, 63, True), (4, 64, 70000, 64, False)]:
        x = gen.make_rejection_inputs(B, N, V, seed, "cuda", tree="eagle", with_q=with_q)
        args = (x.probs, dev(x.draft), dev(x.parents), dev(x.coins, torch.float32),
                dev(x.bonus_u, torch.float32))
        kw = dict(draft_score=dev(x.draft_score, torch.float32),
                  draft_q=x.draft_q if with_q else None)
        fresh = tav.verify_tree_rejection(*args, **kw)
        for rep in range(2):
            got = tav.verify_tree_rejection(*args, **kw, workspace=ws)
            torch.cuda.synchronize()
            for k in ("accepted_path", "accept_len", "accepted_tokens"):
                assert torch.equal(got[k], fresh[k]), (B, N, V, with_q, rep, k)
        assert int(fresh["accept_len"].min()) >= 1
        say("workspace reuse B %d N %d V %d q %s: identical" % (B, N, V, with_q))


def test_rejection_replays_in_a_graph():
    """Both forms captured in a HIP graph with a workspace bound once and
    replayed three times (the call clears its counters with a kernel, so
    every replay starts afresh): each replay equals the eager call."""
    B, N, V = 32, 64, 30000
    for with_q in (False, True):
        x = gen.make_rejection_inputs(B, N, V, 71, "cuda", tree="eagle", with_q=with_q)
        args = (x.probs, dev(x.draft), dev(x.parents), dev(x.coins, torch.float32),
                dev(x.bonus_u, torch.float32))
        kw = dict(draft_score=dev(x.draft_score, torch.float32),
                  draft_q=x.draft_q if with_q else None)
        ws = torch.empty(tav.verify_tree_rejection_workspace_size(B, N, V), dtype=torch.uint8,
                         device="cuda")
        eager = tav.verify_tree_rejection(*args, **kw, workspace=ws)
        torch.cuda.synchronize()
        eager = {k: v.clone() for k, v in eager.items()}
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):     # warm the capture stream first
            tav.verify_tree_rejection(*args, **kw, workspace=ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            got = tav.verify_tree_rejection(*args, **kw, workspace=ws)
        torch.cuda.synchronize()
        for rep in range(3):
            for v in got.values():
                v.fill_(-7)               # every replay must rewrite every output
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for k in eager:
                assert torch.equal(got[k], eager[k]), (with_q, rep, k)
        say("graph replays, q form %s: identical to the eager call" % with_q)
