"""GPU parity of the MLA latent-cache cascade through the C ABI against the
CPU fp64 oracle: out max |err| <= 1e-2, lse2 <= 1e-3, with bf16 latent
caches and with FP8 E4M3 ones (the query rounded to E4M3 for every key).
Reduced sizes check every row (several row groups, split counts and ragged
prefixes); the full MLA workloads, in the benchmark's launch, check sampled
rows and that every output is finite (unseen slots hold NaN)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verify_amd as tav
from tree_attention_verify_amd import inputs as gen

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
LSE_TOL = 1e-3


def say(*a):
    print("[mla]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tav.lib()


def dev(x, dtype=torch.int32):
    return torch.as_tensor(np.ascontiguousarray(x)).to(dtype).cuda()


def run(inp, masks):
    wl = inp.wl
    out, lse = tav.tree_attention_mla(inp.q, inp.latent, dev(inp.page_table), dev(inp.prefix_len),
                                      dev(masks.view(np.int64), torch.int64), wl.W, Dc=wl.Dc,
                                      max_prefix_len=int(inp.prefix_len.max()))
    torch.cuda.synchronize()
    return out, lse


def check(inp, masks, out, lse, rows=None, tag=""):
    wl = inp.wl
    ro, rl = oracle.mla_attention(gen.bf16_bits(inp.q), gen.bf16_bits(inp.latent), inp.strides,
                                  inp.page_table, wl.page_size, inp.prefix_len, masks, wl.W,
                                  wl.Dc, wl.Dr, rows=rows)
    o = out.float().cpu().numpy().reshape(-1, wl.Dc)
    l = lse.cpu().numpy().reshape(-1)
    if rows is not None:
        o, l = o[rows], l[rows]
    assert np.isfinite(o).all() and np.isfinite(l).all(), tag
    err = float(np.abs(o - ro.reshape(o.shape)).max())
    lerr = float(np.abs(l - rl.reshape(l.shape)).max())
    say(tag, "max|out err| %.2e  max|lse2 err| %.2e" % (err, lerr))
    assert err <= OUT_TOL and lerr <= LSE_TOL, (tag, err, lerr)


SMALL = {
    # name: (workload, prefix lengths)
    "rows64": (gen.MlaWorkload("m", 2, 700, 16, 4, 512, 64, 64), [700, 95]),
    "rows128": (gen.MlaWorkload("m", 3, 1000, 8, 16, 512, 64, 16), [1000, 37, 513]),
    "rows512": (gen.MlaWorkload("m", 2, 300, 64, 8, 512, 64, 64), [300, 129]),
    "norope": (gen.MlaWorkload("m", 2, 640, 16, 8, 512, 0, 32), [640, 1]),
    "noprefix": (gen.MlaWorkload("m", 2, 0, 12, 4, 512, 64, 64), [0, 0]),
    "long": (gen.MlaWorkload("m", 1, 9000, 16, 16, 512, 64, 64), [9000]),
    # 80 folded rows (a second, partial 64-row group), pages of 8 keys
    "ragged_rows": (gen.MlaWorkload("m", 2, 1500, 5, 16, 512, 64, 8), [1500, 777]),
    # 15 folded rows, no rotary part, pages of 4 keys, a one-key prefix
    "tiny": (gen.MlaWorkload("m", 3, 200, 5, 3, 512, 0, 4), [200, 33, 1]),
}


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_mla_parity_every_row(name, kv):
    wl, pl = SMALL[name]
    if kv == "fp8":
        wl = wl.with_(kv_dtype="fp8")
    say("case", name, wl)
    inp = gen.make_mla_inputs(wl, 21, "cuda", prefix_lens=np.array(pl))
    m = oracle.build_masks(inp.parents)["masks"]
    out, lse = run(inp, m)
    check(inp, m, out, lse, tag=name + " " + kv)


@pytest.mark.parametrize("name", sorted(gen.MLA_WORKLOADS))
def test_mla_full_size_sampled_rows(name):
    wl = gen.MLA_WORKLOADS[name]
    inp = gen.make_mla_inputs(wl, 4, "cuda")
    m = oracle.build_masks(inp.parents)["masks"]
    out, lse = run(inp, m)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(wl.B * wl.R * wl.Hq, size=24, replace=False))
    check(inp, m, out, lse, rows=rows, tag=name)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_mla_late_dominant_key_repeats_the_pass(kv):
    # Every head's query is all ones and one late prefix key holds 3.0 in
    # every channel (both exact in E4M3): its score passes the first block's
    # row max by far more than 64 (log2 units), so each split holding it is
    # computed again with the exact row max as the reference; the result is
    # still the oracle's.
    wl = gen.MlaWorkload("m", 2, 2000, 8, 16, 512, 64, 64, kv_dtype="" if kv == "bf16" else kv)
    inp = gen.make_mla_inputs(wl, 31, "cuda", prefix_lens=np.array([2000, 1500]))
    inp.q.fill_(1.0)
    for b, t in ((0, 1900), (1, 700)):
        pg = int(inp.page_table[b, t // wl.page_size])
        inp.latent[pg, t % wl.page_size, :] = 3.0
    m = oracle.build_masks(inp.parents)["masks"]
    out, lse = run(inp, m)
    check(inp, m, out, lse, tag="late dominant key")
    # the dominant key's latent part is the output
    assert torch.allclose(out.float(), torch.full_like(out.float(), 3.0), atol=1e-2)


def _same_nonfinite(ours, ref, tol, tag):
    """Element-wise: where the oracle is finite, ours is finite and within tol;
    where it is NaN / +inf / -inf, ours is the same."""
    assert np.array_equal(np.isnan(ours), np.isnan(ref)), tag + ": NaN pattern"
    assert np.array_equal(np.isposinf(ours), np.isposinf(ref)), tag + ": +inf pattern"
    assert np.array_equal(np.isneginf(ours), np.isneginf(ref)), tag + ": -inf pattern"
    fin = np.isfinite(ref)
    if fin.any():
        assert np.abs(ours[fin] - ref[fin]).max() <= tol, tag


def test_mla_nonfinite_window_rows_reach_only_rows_that_see_them():
    # NaN in a latent channel of window node j1, NaN in a rotary channel of
    # j2, +inf in a latent channel of j3 (a score of +inf or -inf depending
    # on the query's sign, and an infinite value channel): a row is
    # non-finite exactly where the exact softmax over its visible keys is
    wl = gen.MlaWorkload("nf", 2, 300, 16, 8, 512, 64, 16)
    inp = gen.make_mla_inputs(wl, 13, "cuda", prefix_lens=np.array([300, 123]))

    def slot(b, j):
        t = int(inp.prefix_len[b]) + j
        return int(inp.page_table[b, t // wl.page_size]), t % wl.page_size

    j1, j2, j3 = 2, 4, 7
    for b in range(wl.B):
        pg, sl = slot(b, j1)
        inp.latent[pg, sl, 17] = float("nan")
        pg, sl = slot(b, j2)
        inp.latent[pg, sl, 512 + 9] = float("nan")
        pg, sl = slot(b, j3)
        inp.latent[pg, sl, 300] = float("inf")
    m = oracle.build_masks(inp.parents)["masks"]
    out, lse = run(inp, m)
    ro, rl = oracle.mla_attention(gen.bf16_bits(inp.q), gen.bf16_bits(inp.latent), inp.strides,
                                  inp.page_table, wl.page_size, inp.prefix_len, m, wl.W, wl.Dc, wl.Dr)
    _same_nonfinite(out.float().cpu().numpy().reshape(ro.shape), ro, OUT_TOL, "mla out")
    _same_nonfinite(lse.cpu().numpy().reshape(rl.shape), rl, LSE_TOL, "mla lse2")
    sees = lambda j: ((m.astype(np.uint64) >> np.uint64(j)) & np.uint64(1)).astype(bool)
    assert sees(j1).any() and sees(j3).any() and (~sees(j1)).any(), "the trees must reach the nodes"
    assert np.isfinite(ro).any() and not np.isfinite(ro).all()


@pytest.mark.parametrize("P", [300, 2000])
def test_mla_nonfinite_prefix_rows(P):
    # request 0: +inf in latent channel 300 of one prefix key (a score of
    # +inf or -inf by the query's sign, and an infinite value channel) and
    # NaN in a rotary channel of another; request 1 clean.  Every row sees
    # the whole prefix, so request 0's rows are non-finite exactly where the
    # exact softmax is, and request 1 stays finite.  P = 2000 runs several
    # splits (the merge combines their partials).
    wl = gen.MlaWorkload("nfp", 2, P, 8, 8, 512, 64, 16)
    inp = gen.make_mla_inputs(wl, 17, "cuda", prefix_lens=np.array([P, P // 2 + 3]))

    def slot(t):
        return int(inp.page_table[0, t // wl.page_size]), t % wl.page_size

    pg, sl = slot(P // 3)
    inp.latent[pg, sl, 300] = float("inf")
    pg, sl = slot(P - 5)
    inp.latent[pg, sl, 512 + 9] = float("nan")
    m = oracle.build_masks(inp.parents)["masks"]
    out, lse = run(inp, m)
    ro, rl = oracle.mla_attention(gen.bf16_bits(inp.q), gen.bf16_bits(inp.latent), inp.strides,
                                  inp.page_table, wl.page_size, inp.prefix_len, m, wl.W, wl.Dc, wl.Dr)
    o = out.float().cpu().numpy().reshape(ro.shape)
    _same_nonfinite(o, ro, OUT_TOL, "mla prefix out")
    _same_nonfinite(lse.cpu().numpy().reshape(rl.shape), rl, LSE_TOL, "mla prefix lse2")
    assert not np.isfinite(ro[0]).all() and np.isfinite(ro[1]).all()
