"""GPU parity: the HIP path (through the C ABI) against the CPU fp64 oracle.

Bars: masks, depth, positions, tree errors, accepted paths, accept lengths,
accepted tokens and compaction bit-exact; attention out max |err| <= 1e-2 and
lse2 max |err| <= 1e-3 against the fp64 oracle on the same bf16-rounded (or
fp32) inputs.  Reduced sizes are checked element by element over every row;
the full workload sizes, in the launch configuration the benchmark times, are
checked on sampled rows plus whole-output properties (finite everywhere).
"""
import math
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
    print("[parity]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tav.lib()  # loud failure if the HIP library is missing


def dev(x, dtype=torch.int32):
    return torch.as_tensor(np.ascontiguousarray(x)).to(dtype).cuda()


def masks_np(t):
    return t.cpu().numpy().view(np.uint64)


def gpu_masks(inp):
    r = tav.tree_build_masks(dev(inp.parents), vc=dev(inp.prefix_len))
    torch.cuda.synchronize()
    return r


def run_attention(inp, masks_dev, prefix_window=None):
    wl = inp.wl
    pw = wl.prefix_window if prefix_window is None else prefix_window
    out, lse = tav.tree_attention(inp.q, inp.k_cache, inp.v_cache, dev(inp.page_table),
                                  dev(inp.prefix_len), masks_dev, wl.W,
                                  max_prefix_len=int(inp.prefix_len.max()), layout=inp.layout,
                                  prefix_window=pw)
    torch.cuda.synchronize()
    return out, lse


def oracle_attention(inp, masks, rows=None, prefix_window=None):
    wl = inp.wl
    pw = wl.prefix_window if prefix_window is None else prefix_window
    return oracle.tree_attention(gen.bf16_bits(inp.q), gen.bf16_bits(inp.k_cache),
                                 gen.bf16_bits(inp.v_cache), inp.strides, inp.page_table,
                                 wl.page_size, inp.prefix_len, masks, wl.W, wl.Hkv,
                                 prefix_window=pw, rows=rows)


def check_attention(out, lse, ref_o, ref_l, rows=None, tag=""):
    o = out.float().cpu().numpy().reshape(-1, out.shape[-1])
    l = lse.cpu().numpy().reshape(-1)
    if rows is not None:
        o, l = o[rows], l[rows]
    ref_o = ref_o.reshape(o.shape)
    ref_l = ref_l.reshape(l.shape)
    assert np.isfinite(o).all(), tag + ": non-finite output"
    err = float(np.abs(o - ref_o).max())
    both_inf = np.isneginf(l) & np.isneginf(ref_l)
    lerr = float(np.abs(np.where(both_inf, 0.0, l - ref_l)).max())
    say(tag, "max|out err| = %.2e  max|lse2 err| = %.2e" % (err, lerr))
    assert err <= OUT_TOL, tag
    assert lerr <= LSE_TOL, tag


# ---------------------------------------------------------------------------
# reduced-size cases: several tiles, ragged tails, every row checked
# ---------------------------------------------------------------------------

W_ = gen.WORKLOADS
SMALL = {
    "worked": (W_["worked"], None),
    "random16": (W_["random16"].with_(B=3, P=1000), [1000, 37, 513]),
    "eagle64": (W_["eagle64"].with_(B=2, P=700), [700, 333]),
    "long64": (W_["long64"].with_(B=2, P=3000), [3000, 2049]),
    "lanes": (W_["lanes"].with_(B=4, P=5000, prefix_window=1000), [5000, 999, 1000, 4500]),
    "chain8": (W_["chain8"].with_(B=4, P=2000), [2000, 1, 64, 1999]),
    "rows128": (W_["random16"].with_(name="rows128", B=2, P=900, N=32), [900, 700]),
    "d64_bf16": (W_["random16"].with_(name="d64", B=2, P=777, N=16, Hq=8, Hkv=2, D=64),
                 [777, 100]),
    "f32_d128": (W_["worked"].with_(name="f32", B=2, P=300, N=8, Hq=8, Hkv=4, D=128,
                                    tree="random", depth_cap=4), [300, 17]),
    # 512 folded rows and one split: the window kernel merges and writes the output
    "onesplit512": (W_["long64"].with_(name="onesplit512", B=2, P=500, N=64, Hq=32, Hkv=4,
                                       page_size=16), [500, 131]),
    # W = 33: a second, mostly empty 32-key window block
    "w33": (W_["random16"].with_(name="w33", B=2, P=640, N=33, depth_cap=5), [640, 90]),
    # FP8 E4M3 K/V caches (bf16 query): every prefix kernel shape and the window
    "fp8_rows64": (W_["random16"].with_(name="fp8_64", B=3, P=1000, kv_dtype="fp8"),
                   [1000, 37, 513]),
    "fp8_chain8": (W_["chain8"].with_(name="fp8_chain", B=4, P=2000, kv_dtype="fp8"),
                   [2000, 1, 64, 1999]),
    "fp8_lanes": (W_["lanes"].with_(name="fp8_lanes", B=4, P=5000, prefix_window=1000,
                                    kv_dtype="fp8"), [5000, 999, 1000, 4500]),
    "fp8_rows128": (W_["random16"].with_(name="fp8_128", B=2, P=900, N=32, kv_dtype="fp8"),
                    [900, 700]),
    "fp8_long64": (W_["long64"].with_(name="fp8_long", B=2, P=3000, kv_dtype="fp8"),
                   [3000, 2049]),
    "fp8_onesplit512": (W_["long64"].with_(name="fp8_one", B=2, P=500, N=64, Hq=32, Hkv=4,
                                           page_size=16, kv_dtype="fp8"), [500, 131]),
    "fp8_d64": (W_["random16"].with_(name="fp8_d64", B=2, P=777, N=16, Hq=8, Hkv=2, D=64,
                                     kv_dtype="fp8"), [777, 100]),
    # one 8-way tensor-parallel share of long64: one kv head, 4 query heads
    "long64_tp8": (W_["long64_tp8"].with_(B=2, P=3000), [3000, 2049]),
    # 64-channel heads with 256 folded rows (the wide-row kernel at D = 64)
    "d64_rows256": (W_["random16"].with_(name="d64w", B=2, P=1111, N=64, Hq=8, Hkv=2, D=64,
                                         depth_cap=8), [1111, 250]),
}


@pytest.fixture(scope="module", params=sorted(SMALL))
def small(request):
    name = request.param
    wl, pl = SMALL[name]
    say("case", name, wl)
    inp = gen.make_inputs(wl, 11, "cuda", prefix_lens=pl)
    return name, inp


def test_masks_bit_exact(small):
    name, inp = small
    if inp.wl.tree == "lanes":
        pytest.skip("lane masks are drafter inputs")
    g = gpu_masks(inp)
    r = oracle.build_masks(inp.parents, vc=inp.prefix_len)
    assert np.array_equal(masks_np(g["masks"]), r["masks"])
    assert np.array_equal(g["depth"].cpu().numpy(), r["depth"])
    assert np.array_equal(g["positions"].cpu().numpy(), r["positions"])
    assert np.array_equal(g["tree_error"].cpu().numpy(), r["tree_error"])


def test_greedy_bit_exact(small):
    name, inp = small
    if inp.wl.tree == "lanes":
        pytest.skip("no verify for draft lanes")
    g = tav.verify_tree_greedy(dev(inp.draft), dev(inp.target), dev(inp.parents))
    r = oracle.verify_greedy(inp.draft, inp.target, inp.parents)
    for k in ("accepted_path", "accept_len", "accepted_tokens"):
        assert np.array_equal(g[k].cpu().numpy(), r[k]), k


def test_attention_parity(small):
    name, inp = small
    if inp.wl.tree == "lanes":
        m_np = inp.lane_masks
        m_dev = dev(m_np.view(np.int64), torch.int64)
    else:
        g = gpu_masks(inp)
        m_dev = g["masks"]
        m_np = oracle.build_masks(inp.parents)["masks"]
    out, lse = run_attention(inp, m_dev)
    ro, rl = oracle_attention(inp, m_np)
    check_attention(out, lse, ro, rl, tag=name)


def test_compaction_bit_exact(small):
    name, inp = small
    if inp.wl.tree == "lanes":
        pytest.skip("no verify for draft lanes")
    wl = inp.wl
    g = tav.verify_tree_greedy(dev(inp.draft), dev(inp.target), dev(inp.parents))
    r = oracle.verify_greedy(inp.draft, inp.target, inp.parents)
    hidden = torch.randint(-2**31, 2**31 - 1, (wl.B, wl.N, 72), dtype=torch.int32,
                           device="cuda")
    kc, vc, hc = (inp.k_cache.cpu().clone(), inp.v_cache.cpu().clone(), hidden.cpu().clone())
    pt = dev(inp.page_table)
    pl = dev(inp.prefix_len)
    tables = [tav.RowTable.paged_kv(inp.k_cache, pt, pl, inp.layout),
              tav.RowTable.paged_kv(inp.v_cache, pt, pl, inp.layout),
              tav.RowTable.dense_rows(hidden)]
    tav.compact_window_rows(tables, g["accepted_path"], g["accept_len"])
    torch.cuda.synchronize()
    host_tables = []
    for t, buf in zip(tables, (kc, vc, hc)):
        nb = buf.view(torch.uint8).numpy() if buf.dtype != torch.bfloat16 else \
            buf.view(torch.int16).numpy().view(np.uint8)
        host_tables.append(dict(buf=nb, page_table=None if t.page_table is None else inp.page_table,
                                prefix_len=None if t.page_table is None else inp.prefix_len,
                                page_size=t.page_size, stride_page=t.stride_page,
                                stride_token=t.stride_token, stride_head=t.stride_head,
                                stride_batch=t.stride_batch, n_heads=t.n_heads,
                                row_bytes=t.row_bytes))
    oracle.compact_rows(host_tables, r["accepted_path"], r["accept_len"])
    for t, h in zip(tables, host_tables):
        got = t.buf.cpu().contiguous()
        got = got.view(torch.int16).numpy().view(np.uint8) if got.dtype == torch.bfloat16 \
            else got.view(torch.uint8).numpy()
        assert np.array_equal(got, h["buf"]), "compaction differs"


def test_shift_bit_exact(small):
    name, inp = small
    if inp.wl.tree == "lanes":
        pytest.skip("no positions for draft lanes")
    g = gpu_masks(inp)
    depth = g["depth"].cpu().numpy()
    chain = inp.prefix_len[:, None] + np.arange(inp.wl.N, dtype=np.int32)[None]
    p = dev(chain)
    tav.tree_shift_positions(p, g["depth"], +1)
    torch.cuda.synchronize()
    up = oracle.shift_positions(chain, depth, +1)
    assert np.array_equal(p.cpu().numpy(), up)
    assert np.array_equal(up, g["positions"].cpu().numpy())
    tav.tree_shift_positions(p, g["depth"], -1)
    torch.cuda.synchronize()
    assert np.array_equal(p.cpu().numpy(), chain)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_short_and_empty_prefixes(dtype):
    pl = [0, 1, 15, 16, 17, 63, 64, 65]
    wl = gen.Workload("edge", len(pl), 65, 8, 8, 2, 128, dtype, 16, "random", depth_cap=3)
    inp = gen.make_inputs(wl, 3, "cuda", prefix_lens=pl)
    g = gpu_masks(inp)
    out, lse = run_attention(inp, g["masks"])
    ro, rl = oracle_attention(inp, oracle.build_masks(inp.parents)["masks"])
    check_attention(out, lse, ro, rl, tag="short-prefix-" + dtype)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("rows", [32, 64, 256])
@pytest.mark.parametrize("ps", [1, 2, 4])
def test_small_pages(ps, rows, kv):
    # pages of fewer than 8 keys: the loads look up a page per lane (every
    # prefix kernel shape: 32, 64 and 256 folded rows)
    n, hq = {32: (8, 8), 64: (16, 8), 256: (64, 8)}[rows]
    wl = gen.Workload("sp", 2, 300, n, hq, 2, 128, "bf16", ps, "random", depth_cap=5, kv_dtype=kv)
    inp = gen.make_inputs(wl, 20 + ps, "cuda", prefix_lens=[300, 77])
    m = oracle.build_masks(inp.parents)["masks"]
    out, lse = run_attention(inp, dev(m.view(np.int64), torch.int64))
    ro, rl = oracle_attention(inp, m)
    check_attention(out, lse, ro, rl, tag="pages of %d, %d rows, %s" % (ps, rows, kv))


def test_nhd_layout_and_high_mask_bits():
    wl = gen.Workload("nhd", 2, 300, 12, 16, 4, 128, "bf16", 16, "random", depth_cap=5)
    inp = gen.make_inputs(wl, 4, "cuda", layout="NHD", prefix_lens=[300, 123])
    m = oracle.build_masks(inp.parents)["masks"]
    noisy = m | (np.uint64(0xFFFF) << np.uint64(48))        # bits >= W must be ignored
    out, lse = run_attention(inp, dev(noisy.view(np.int64), torch.int64))
    ro, rl = oracle_attention(inp, m)
    check_attention(out, lse, ro, rl, tag="NHD")


PHASE_SHAPES = {
    # 512 folded rows, one split: the prefix launch takes the window keys and
    # writes the output, the window-and-merge phase launches nothing
    "pipe_one_split": gen.Workload("ph1", 2, 300, 64, 16, 2, 128, "bf16", 16, "random", depth_cap=6),
    # 256 folded rows, several splits: prefix partials, then window and merge
    "pipe_splits": gen.Workload("ph2", 2, 3000, 64, 32, 8, 128, "bf16", 64, "random", depth_cap=8),
    # 64 folded rows (the small-row prefix kernel)
    "small_rows": gen.Workload("ph3", 3, 700, 16, 32, 8, 128, "bf16", 16, "random", depth_cap=6),
    # 32 folded rows, one split (the window in the prefix launch)
    "rows32_one_split": gen.Workload("ph4", 2, 300, 8, 8, 2, 128, "bf16", 16, "random", depth_cap=5),
}


@pytest.mark.parametrize("shape", sorted(PHASE_SHAPES))
def test_phases_equal_one_call(shape):
    # tree_attention is exactly tree_attention_prefix then
    # tree_attention_window_merge with the same arguments: bit for bit, and
    # both within the bars of the oracle
    wl = PHASE_SHAPES[shape]
    say("case", shape, wl)
    inp = gen.make_inputs(wl, 12, "cuda")
    m = oracle.build_masks(inp.parents)["masks"]
    md = dev(m.view(np.int64), torch.int64)
    out1, lse1 = run_attention(inp, md)
    kw = dict(max_prefix_len=int(inp.prefix_len.max()), layout=inp.layout,
              prefix_window=wl.prefix_window)
    args = (inp.q, inp.k_cache, inp.v_cache, dev(inp.page_table), dev(inp.prefix_len), md, wl.W)
    out2 = torch.full_like(inp.q, float("nan"))
    lse2 = torch.full_like(lse1, float("nan"))
    ws = torch.empty(tav.tree_attention_workspace_size(inp.q.dtype, wl.B, wl.R, wl.Hq, wl.Hkv, wl.D,
                                                       kw["max_prefix_len"], wl.prefix_window,
                                                       wl.page_size),
                     dtype=torch.uint8, device="cuda")
    tav.tree_attention(*args, **kw, out=out2, lse2=lse2, workspace=ws, phase="prefix")
    tav.tree_attention(*args, **kw, out=out2, lse2=lse2, workspace=ws, phase="window_merge")
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16)), shape + ": out"
    assert torch.equal(lse1.view(torch.int32), lse2.view(torch.int32)), shape + ": lse2"
    ro, rl = oracle_attention(inp, m)
    check_attention(out1, lse1, ro, rl, tag=shape)


ONE_SPLIT_CASES = {
    # (workload, prefix lengths or None, layout): every case runs the kernel for
    # more than 128 folded rows as one split, so its prefix launch takes the
    # window keys and writes the output
    "d64": (gen.Workload("os1", 2, 300, 64, 16, 2, 64, "bf16", 16, "random", depth_cap=6), None, "HND"),
    "empty_prefix": (gen.Workload("os2", 3, 500, 40, 16, 2, 128, "bf16", 16, "random", depth_cap=5),
                     [500, 0, 37], "HND"),
    "sliding": (gen.Workload("os3", 2, 2000, 64, 16, 2, 128, "bf16", 64, "random", depth_cap=8,
                             prefix_window=200), None, "HND"),
    "pages1": (gen.Workload("os4", 1, 300, 17, 32, 4, 128, "bf16", 1, "random", depth_cap=4), None, "HND"),
    "pages2_nhd": (gen.Workload("os5", 2, 400, 33, 16, 2, 128, "bf16", 2, "random", depth_cap=5),
                   [400, 251], "NHD"),
    # the kernel for at most 32 folded rows, one split
    "rows32": (gen.Workload("os6", 2, 300, 8, 8, 2, 128, "bf16", 16, "random", depth_cap=5), None, "HND"),
    "rows16_d64_empty": (gen.Workload("os7", 3, 400, 4, 8, 2, 64, "bf16", 2, "random", depth_cap=3),
                         [400, 0, 9], "HND"),
    "rows32_sliding_nhd": (gen.Workload("os8", 2, 3000, 8, 16, 4, 128, "bf16", 64, "random", depth_cap=6,
                                        prefix_window=150), None, "NHD"),
}


@pytest.mark.parametrize("case", sorted(ONE_SPLIT_CASES))
def test_one_split_window_in_prefix_launch(case):
    # the prefix phase alone writes the output (so the fused path is the one
    # that ran), and every row matches the oracle
    wl, lens, layout = ONE_SPLIT_CASES[case]
    say("case", case, wl)
    inp = gen.make_inputs(wl, 21, "cuda", layout=layout,
                          prefix_lens=None if lens is None else np.array(lens, np.int32))
    m = oracle.build_masks(inp.parents)["masks"]
    md = dev(m.view(np.int64), torch.int64)
    out = torch.full_like(inp.q, float("nan"))
    lse = torch.full((wl.B, wl.R, wl.Hq), float("nan"), dtype=torch.float32, device="cuda")
    tav.tree_attention(inp.q, inp.k_cache, inp.v_cache, dev(inp.page_table), dev(inp.prefix_len), md,
                       wl.W, max_prefix_len=int(inp.prefix_len.max()), layout=layout,
                       prefix_window=wl.prefix_window, out=out, lse2=lse, phase="prefix")
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any(), case + ": the prefix launch did not write the output"
    ro, rl = oracle_attention(inp, m)
    check_attention(out, lse, ro, rl, tag=case)


MANY_SPLIT_CASES = {
    # (workload, prefix lengths, bounds on the partials per row S): one kv head,
    # so the prefix runs many splits, and the merge shares each row among 4
    # (16 < S <= 64) or 8 (S > 64) waves; the second request is shorter, so
    # its last splits are empty
    "pipe_s95": (gen.Workload("ms1", 2, 30000, 64, 4, 1, 128, "bf16", 64, "random", depth_cap=8),
                 [30000, 17001], (65, 10**9)),
    "pipe_s39": (gen.Workload("ms2", 2, 12000, 64, 4, 1, 128, "bf16", 64, "random", depth_cap=8),
                 [12000, 5000], (17, 64)),
    "rows64_d64_s80": (gen.Workload("ms3", 2, 50000, 16, 4, 1, 64, "bf16", 16, "random", depth_cap=5),
                       [50000, 20001], (65, 10**9)),
    "rows64_d64_s20": (gen.Workload("ms4", 2, 12000, 16, 4, 1, 64, "bf16", 16, "random", depth_cap=5),
                       [12000, 777], (17, 64)),
    "fp8_pipe_s39": (gen.Workload("ms5", 2, 12000, 64, 4, 1, 128, "bf16", 64, "random", depth_cap=8,
                                  kv_dtype="fp8"), [12000, 5000], (17, 64)),
    # more than 128 partials: each of the 8 waves takes several rounds and
    # rescales its sums when a later round raises its max
    "pipe_s220": (gen.Workload("ms6", 1, 70000, 64, 4, 1, 128, "bf16", 64, "random", depth_cap=8),
                  [70000], (129, 10**9)),
    "rows64_d64_s158": (gen.Workload("ms7", 1, 100000, 16, 4, 1, 64, "bf16", 16, "random", depth_cap=5),
                        [100000], (129, 10**9)),
}


@pytest.mark.parametrize("case", sorted(MANY_SPLIT_CASES))
def test_many_split_merge(case):
    wl, pl, (s_lo, s_hi) = MANY_SPLIT_CASES[case]
    say("case", case, wl, pl)
    inp = gen.make_inputs(wl, 21, "cuda", prefix_lens=pl)
    # the partial count the plan gives, read back from the workspace size
    rows = wl.B * wl.R * wl.Hq
    nbytes = tav.tree_attention_workspace_size(inp.q.dtype, wl.B, wl.R, wl.Hq, wl.Hkv, wl.D,
                                               int(inp.prefix_len.max()), wl.prefix_window,
                                               wl.page_size, inp.k_cache.dtype)
    S = nbytes // (rows * (wl.D + 1) * 4)
    assert s_lo <= S <= s_hi, (case, S)
    m = oracle.build_masks(inp.parents)["masks"]
    out, lse = run_attention(inp, dev(m.view(np.int64), torch.int64))
    ro, rl = oracle_attention(inp, m)
    check_attention(out, lse, ro, rl, tag="%s (S %d)" % (case, S))


# Few splits: with one prefix partial (S = 2 with the window's) the window
# kernel merges it itself, with more the merge kernel runs.  Two requests
# over 8 kv heads leave room for 16 splits, so P = 512 k gives k splits of
# the 64-row kernel (four 128-key stages each) and S = k + 1.
FEW_SPLIT_CASES = {
    "rows64_s%d" % (k + 1): (gen.Workload("fs%d" % k, 2, 512 * k, 16, 32, 8, 128, "bf16", 16,
                                          "random", depth_cap=6), k + 1)
    for k in (1, 2, 3, 4, 5)
}
FEW_SPLIT_CASES.update({
    "fp8_rows64_s4": (gen.Workload("fs_fp8", 2, 1536, 16, 32, 8, 128, "bf16", 16, "random",
                                   depth_cap=6, kv_dtype="fp8"), 4),
    "d64_rows64_s3": (gen.Workload("fs_d64", 2, 1024, 16, 32, 8, 64, "bf16", 16, "random",
                                   depth_cap=6), 3),
    # 256 folded rows (the pipelined kernel): 64-key stages, 3 splits
    "rows256_s4": (gen.Workload("fs_pipe", 2, 768, 64, 32, 8, 128, "bf16", 64, "random",
                                depth_cap=8), 4),
})


def _partials_per_row(inp):
    wl = inp.wl
    nbytes = tav.tree_attention_workspace_size(inp.q.dtype, wl.B, wl.R, wl.Hq, wl.Hkv, wl.D,
                                               int(inp.prefix_len.max()), wl.prefix_window,
                                               wl.page_size, inp.k_cache.dtype)
    return nbytes // (wl.B * wl.R * wl.Hq * (wl.D + 1) * 4)


@pytest.mark.parametrize("case", sorted(FEW_SPLIT_CASES))
def test_few_split_merge(case):
    wl, S_want = FEW_SPLIT_CASES[case]
    P = wl.P
    inp = gen.make_inputs(wl, 23, "cuda", prefix_lens=[P, P // 3 + 5])
    S = _partials_per_row(inp)
    say("case", case, wl, "S", S)
    assert S == S_want, (case, S)
    m = oracle.build_masks(inp.parents)["masks"]
    out, lse = run_attention(inp, dev(m.view(np.int64), torch.int64))
    ro, rl = oracle_attention(inp, m)
    check_attention(out, lse, ro, rl, tag="%s (S %d)" % (case, S))


@pytest.mark.parametrize("k", [2, 5])
def test_nonfinite_prefix_values_through_the_merge(k):
    # request 0, kv head 0: NaN in one prefix key's K, and in prefix V channel
    # 77 one +inf and one -inf (NaN) and in channel 5 one +inf (+inf), in
    # different splits; every row of that head sees every prefix key, so the
    # whole head is NaN (the NaN key) -- with the K NaN left out, channel 77
    # is NaN, channel 5 +inf and the rest finite.  The merge kernel combines
    # the S = 3 and S = 6 partials of a row.
    wl = FEW_SPLIT_CASES["rows64_s%d" % (k + 1)][0]
    for with_k_nan in (False, True):
        inp = gen.make_inputs(wl, 29, "cuda", prefix_lens=[wl.P, wl.P // 3 + 5])
        assert _partials_per_row(inp) == k + 1

        def slot(t):
            return int(inp.page_table[0, t // wl.page_size]), t % wl.page_size

        P0 = int(inp.prefix_len[0])
        pg, sl = slot(3)
        inp.v_cache[pg, 0, sl, 77] = float("inf")
        pg, sl = slot(P0 - 2)
        inp.v_cache[pg, 0, sl, 77] = float("-inf")
        pg, sl = slot(P0 // 2)
        inp.v_cache[pg, 0, sl, 5] = float("inf")
        if with_k_nan:
            pg, sl = slot(P0 // 3)
            inp.k_cache[pg, 0, sl] = float("nan")
        m = oracle.build_masks(inp.parents)["masks"]
        out, lse = run_attention(inp, dev(m.view(np.int64), torch.int64))
        ro, rl = oracle_attention(inp, m)
        tag = "S %d, K NaN %s" % (k + 1, with_k_nan)
        o = out.float().cpu().numpy()
        _same_nonfinite(o, ro.reshape(out.shape), OUT_TOL, tag + " out")
        _same_nonfinite(lse.cpu().numpy(), rl.reshape(lse.shape), LSE_TOL, tag + " lse2")
        G = wl.Hq // wl.Hkv
        head0 = o[0, :, :G]
        if with_k_nan:
            assert np.isnan(head0).all(), tag
        else:
            assert np.isnan(head0[..., 77]).all() and np.isposinf(head0[..., 5]).all(), tag
        assert np.isfinite(o[1]).all() and np.isfinite(o[0, :, G:]).all(), tag


# A split whose last stage is partial leaves the stage rows past its end
# unloaded; with more stages than stage buffers those rows hold an earlier
# stage's keys.  Their weight is exactly 0, so a +-inf V value there must not
# turn into 0 * inf = NaN: prefix key 150 carries +inf in channel 5, the
# stage ring brings it back into the unloaded rows of the last stage, and
# every row of kv head 0 must still read +inf there (as the oracle does).
STALE_ROW_CASES = {
    # 256 folded rows (pipelined kernel, one split: window in the same launch),
    # 64-key stages in 4 buffers, 401 keys: stage 6 reuses stage 2's buffer
    "rows256": gen.Workload("stale256", 1, 401, 64, 32, 8, 128, "bf16", 16, "random", depth_cap=8),
    # 64 folded rows: 128-key stages in 2 buffers, stage 3 reuses stage 1's
    "rows64": gen.Workload("stale64", 1, 401, 16, 32, 8, 128, "bf16", 16, "random", depth_cap=6),
    # 32 folded rows (2-wave workgroups): 64-key stages in 2 buffers
    "rows32": gen.Workload("stale32", 1, 209, 8, 32, 8, 128, "bf16", 16, "chain"),
}


@pytest.mark.parametrize("case", sorted(STALE_ROW_CASES))
def test_inf_values_in_reused_stage_rows(case):
    wl = STALE_ROW_CASES[case]
    inp = gen.make_inputs(wl, 31, "cuda")
    key = 150 if case != "rows32" else 90
    pg = int(inp.page_table[0, key // wl.page_size])
    inp.v_cache[pg, 0, key % wl.page_size, 5] = float("inf")
    m = oracle.build_masks(inp.parents)["masks"]
    out, lse = run_attention(inp, dev(m.view(np.int64), torch.int64))
    ro, rl = oracle_attention(inp, m)
    o = out.float().cpu().numpy()
    _same_nonfinite(o, ro.reshape(out.shape), OUT_TOL, case + " out")
    _same_nonfinite(lse.cpu().numpy(), rl.reshape(lse.shape), LSE_TOL, case + " lse2")
    G = wl.Hq // wl.Hkv
    assert np.isposinf(o[0, :, :G, 5]).all(), case


@pytest.mark.parametrize("case", ["rows256", "rows64", "rows32", "rows64_s3"])
def test_inf_prefix_key(case):
    # +inf in channel 0 of one prefix key of kv head 0: rows whose query
    # channel 0 is positive score it +inf (the exact softmax is NaN, lse2 NaN),
    # rows with a negative one -inf (the key weighs 0, the rest is finite)
    wl = (STALE_ROW_CASES[case] if case in STALE_ROW_CASES
          else FEW_SPLIT_CASES["rows64_s3"][0])
    inp = gen.make_inputs(wl, 37, "cuda")
    key = 100
    pg = int(inp.page_table[0, key // wl.page_size])
    inp.k_cache[pg, 0, key % wl.page_size, 0] = float("inf")
    m = oracle.build_masks(inp.parents)["masks"]
    out, lse = run_attention(inp, dev(m.view(np.int64), torch.int64))
    ro, rl = oracle_attention(inp, m)
    _same_nonfinite(out.float().cpu().numpy(), ro.reshape(out.shape), OUT_TOL, case + " out")
    _same_nonfinite(lse.cpu().numpy(), rl.reshape(lse.shape), LSE_TOL, case + " lse2")
    assert np.isnan(rl).any() and np.isfinite(rl).any(), "the plant must reach both kinds of rows"


@pytest.mark.parametrize("case", ["rows256", "rows64", "rows32"])
@pytest.mark.parametrize("what", ["k", "v"])
def test_fp8_nan_prefix_values(case, what):
    # FP8 E4M3 caches hold NaN but no infinities: NaN in channel 5 of one
    # prefix key's K (every row of kv head 0 NaN) or V (channel 5 of those
    # rows NaN); the other heads stay finite
    wl = STALE_ROW_CASES[case].with_(kv_dtype="fp8")
    inp = gen.make_inputs(wl, 41, "cuda")
    key = 150 if case != "rows32" else 90
    pg = int(inp.page_table[0, key // wl.page_size])
    cache = inp.k_cache if what == "k" else inp.v_cache
    cache[pg, 0, key % wl.page_size, 5] = float("nan")
    m = oracle.build_masks(inp.parents)["masks"]
    out, lse = run_attention(inp, dev(m.view(np.int64), torch.int64))
    ro, rl = oracle_attention(inp, m)
    o = out.float().cpu().numpy()
    _same_nonfinite(o, ro.reshape(out.shape), OUT_TOL, case + " out")
    _same_nonfinite(lse.cpu().numpy(), rl.reshape(lse.shape), LSE_TOL, case + " lse2")
    G = wl.Hq // wl.Hkv
    if what == "k":
        assert np.isnan(o[0, :, :G]).all(), case
    else:
        assert np.isnan(o[0, :, :G, 5]).all(), case
    assert np.isfinite(o[0, :, G:]).all(), case


@pytest.mark.parametrize("case", ["rows256", "rows64", "rows32", "rows64_s3"])
def test_inf_window_key(case):
    # +inf in channel 0 of window node 2's K: a row that sees the node and
    # whose query channel 0 is positive scores it +inf (the exact softmax is
    # NaN, lse2 NaN); a negative one gives -inf (the node weighs 0); rows that
    # do not see it are untouched
    wl = (STALE_ROW_CASES[case] if case in STALE_ROW_CASES
          else FEW_SPLIT_CASES["rows64_s3"][0])
    inp = gen.make_inputs(wl, 43, "cuda")
    t = int(inp.prefix_len[0]) + 2
    pg = int(inp.page_table[0, t // wl.page_size])
    inp.k_cache[pg, 0, t % wl.page_size, 0] = float("inf")
    m = oracle.build_masks(inp.parents)["masks"]
    out, lse = run_attention(inp, dev(m.view(np.int64), torch.int64))
    ro, rl = oracle_attention(inp, m)
    _same_nonfinite(out.float().cpu().numpy(), ro.reshape(out.shape), OUT_TOL, case + " out")
    _same_nonfinite(lse.cpu().numpy(), rl.reshape(lse.shape), LSE_TOL, case + " lse2")
    assert np.isnan(rl).any() and np.isfinite(rl).any(), "the plant must reach both kinds of rows"


def test_nan_in_node_leaks_only_to_descendants():
    wl = gen.Workload("nan", 1, 200, 16, 8, 2, 128, "bf16", 16, "random", depth_cap=4)
    inp = gen.make_inputs(wl, 5, "cuda")
    j = 6
    t = int(inp.prefix_len[0]) + j
    pg = int(inp.page_table[0, t // wl.page_size])
    inp.k_cache[pg, 0, t % wl.page_size] = float("nan")
    m = oracle.build_masks(inp.parents)["masks"]
    out, lse = run_attention(inp, dev(m.view(np.int64), torch.int64))
    ro, rl = oracle_attention(inp, m)
    o = out.float().cpu().numpy()
    G = wl.Hq // wl.Hkv
    for r in range(wl.R):
        sees = (int(m[0, r]) >> j) & 1
        for h in range(wl.Hq):
            if sees and h // G == 0:
                assert not np.isfinite(o[0, r, h]).all()
            else:
                assert np.isfinite(o[0, r, h]).all()
                assert np.abs(o[0, r, h] - ro[0, r, h]).max() <= OUT_TOL


def _same_nonfinite(ours, ref, tol, tag):
    """Element-wise: where the oracle is finite, ours is finite and within tol;
    where it is NaN / +inf / -inf, ours is the same."""
    assert np.array_equal(np.isnan(ours), np.isnan(ref)), tag + ": NaN pattern"
    assert np.array_equal(np.isposinf(ours), np.isposinf(ref)), tag + ": +inf pattern"
    assert np.array_equal(np.isneginf(ours), np.isneginf(ref)), tag + ": -inf pattern"
    fin = np.isfinite(ref)
    if fin.any():
        assert np.abs(ours[fin] - ref[fin]).max() <= tol, tag


@pytest.mark.parametrize("shape", ["rows24", "rows64", "rows512"])
def test_nonfinite_window_values_reach_only_rows_that_see_them(shape):
    # window K NaN at node j1, V NaN at one channel of j2, V +inf and -inf at
    # one channel of j3 and j4: a row is non-finite exactly where the exact
    # softmax over its own visible keys is (rows24 and rows512 run as one
    # split, with the window in the prefix launch)
    if shape == "rows24":
        wl = gen.Workload("nfw", 1, 200, 12, 4, 2, 128, "bf16", 16, "random", depth_cap=4)
    elif shape == "rows64":
        wl = gen.Workload("nfw", 1, 200, 16, 8, 2, 128, "bf16", 16, "random", depth_cap=4)
    else:
        wl = gen.Workload("nfw", 2, 300, 64, 16, 2, 128, "bf16", 16, "random", depth_cap=6)
    inp = gen.make_inputs(wl, 9, "cuda")

    def slot(j):
        t = int(inp.prefix_len[0]) + j
        return int(inp.page_table[0, t // wl.page_size]), t % wl.page_size

    j1, j2, j3, j4 = 3, 5, 6, 9
    pg, sl = slot(j1)
    inp.k_cache[pg, 0, sl] = float("nan")
    pg, sl = slot(j2)
    inp.v_cache[pg, 0, sl, 5] = float("nan")
    pg, sl = slot(j3)
    inp.v_cache[pg, 0, sl, 77] = float("inf")
    pg, sl = slot(j4)
    inp.v_cache[pg, 0, sl, 77] = float("-inf")
    m = oracle.build_masks(inp.parents)["masks"]
    out, lse = run_attention(inp, dev(m.view(np.int64), torch.int64))
    ro, rl = oracle_attention(inp, m)
    _same_nonfinite(out.float().cpu().numpy(), ro.reshape(out.shape), OUT_TOL, shape + " out")
    _same_nonfinite(lse.cpu().numpy(), rl.reshape(lse.shape), LSE_TOL, shape + " lse2")
    sees = lambda j: ((m[0].astype(np.uint64) >> np.uint64(j)) & np.uint64(1)).astype(bool)
    assert sees(j1).any() and sees(j2).any() and sees(j3).any(), "the tree must reach the poisoned nodes"


@pytest.mark.parametrize("shape", ["rows64", "rows512"])
def test_fp8_nonfinite_window_values(shape):
    # FP8 E4M3 caches hold NaN but no infinities: NaN in window K at node j1
    # and in one V channel at node j2
    if shape == "rows64":
        wl = gen.Workload("nf8", 1, 200, 16, 8, 2, 128, "bf16", 16, "random", depth_cap=4,
                          kv_dtype="fp8")
    else:
        wl = gen.Workload("nf8", 2, 300, 64, 16, 2, 128, "bf16", 16, "random", depth_cap=6,
                          kv_dtype="fp8")
    inp = gen.make_inputs(wl, 13, "cuda")
    j1, j2 = 2, 7
    for j, cache, ch in ((j1, inp.k_cache, None), (j2, inp.v_cache, 33)):
        t = int(inp.prefix_len[0]) + j
        pg, sl = int(inp.page_table[0, t // wl.page_size]), t % wl.page_size
        if ch is None:
            cache[pg, 0, sl] = float("nan")
        else:
            cache[pg, 0, sl, ch] = float("nan")
    m = oracle.build_masks(inp.parents)["masks"]
    out, lse = run_attention(inp, dev(m.view(np.int64), torch.int64))
    ro, rl = oracle_attention(inp, m)
    _same_nonfinite(out.float().cpu().numpy(), ro.reshape(out.shape), OUT_TOL, shape + " fp8 out")
    _same_nonfinite(lse.cpu().numpy(), rl.reshape(lse.shape), LSE_TOL, shape + " fp8 lse2")


@pytest.mark.parametrize("shape", ["rows16", "rows64", "rows256"])
def test_fp8_prefix_query_cast(shape):
    # Query values that E4M3 cannot hold, all rounding down by 1/17 (ties to
    # the even code: 1.0625 -> 1, 2.125 -> 2, 0.53125 -> 0.5, 4.25 -> 4), and
    # keys with their sign bit cleared, so every score shifts the same way:
    # the prefix scores use the rounded query and the window scores the bf16
    # query.  Scoring the prefix with the bf16 query, or the window with the
    # rounded one, is then far outside the tolerance.  Every prefix kernel
    # shape: 16, 64 and 256 folded rows.
    R, Hq = {"rows16": (4, 4), "rows64": (16, 4), "rows256": (64, 4)}[shape]
    wl = gen.Workload("q8", 2, 700, R, Hq, 1, 128, "bf16", 16, "random", depth_cap=5,
                      kv_dtype="fp8")
    inp = gen.make_inputs(wl, 17, "cuda")
    vals = torch.tensor([1.0625, 2.125, 0.53125, 4.25], dtype=torch.bfloat16, device="cuda")
    idx = torch.randint(0, 4, inp.q.shape, generator=torch.Generator("cuda").manual_seed(5),
                        device="cuda")
    inp.q.copy_(vals[idx])
    inp.k_cache.view(torch.uint8).bitwise_and_(0x7F)
    m = oracle.build_masks(inp.parents)["masks"]
    out, lse = run_attention(inp, dev(m.view(np.int64), torch.int64))
    ro, rl = oracle_attention(inp, m)
    check_attention(out, lse, ro, rl, tag=shape + " fp8 q cast")
    # the other readings, from caches widened to bf16 (exact): the bf16 query
    # on every key, and the rounded query on every key
    k16, v16 = inp.k_cache.to(torch.bfloat16), inp.v_cache.to(torch.bfloat16)
    q8 = inp.q.float().to(torch.float8_e4m3fn).to(torch.bfloat16)
    got = lse.cpu().numpy()
    for qq in (inp.q, q8):
        alt = oracle.tree_attention(gen.bf16_bits(qq), gen.bf16_bits(k16), gen.bf16_bits(v16),
                                    inp.strides, inp.page_table, wl.page_size, inp.prefix_len,
                                    m, wl.W, wl.Hkv)
        assert np.abs(got - alt[1].reshape(got.shape)).max() > 5 * LSE_TOL


def test_bad_trees_flagged():
    par = np.array([[-1, 0, 0, 1, 2, 3, 4, 5],
                    [-1, 0, 5, 1, 2, 3, 4, 5],      # forward reference at node 2
                    [0, 0, 1, 2, 3, 4, 5, 6],       # no root
                    [-1, 0, 1, 2, -1, 4, 5, 6]], np.int32)  # second root at node 4
    vc = np.array([10, 20, 30, 40], np.int32)
    g = tav.tree_build_masks(dev(par), vc=dev(vc))
    torch.cuda.synchronize()
    r = oracle.build_masks(par, vc=vc)
    assert r["tree_error"].tolist() == [0, 3, 1, 5]
    assert np.array_equal(g["tree_error"].cpu().numpy(), r["tree_error"])
    assert np.array_equal(masks_np(g["masks"]), r["masks"])
    assert np.array_equal(g["depth"].cpu().numpy(), r["depth"])
    assert np.array_equal(g["positions"].cpu().numpy(), r["positions"])


def test_greedy_ties_and_width():
    rng = np.random.default_rng(0)
    B, N = 64, 64
    par = np.stack([gen.random_tree(rng, N, int(rng.integers(1, 12))) for _ in range(B)])
    draft = rng.integers(0, 3, (B, N)).astype(np.int32)    # many equal sibling tokens
    target = rng.integers(0, 3, (B, N)).astype(np.int32)
    g = tav.verify_tree_greedy(dev(draft), dev(target), dev(par))
    r = oracle.verify_greedy(draft, target, par)
    for k in ("accepted_path", "accept_len", "accepted_tokens"):
        assert np.array_equal(g[k].cpu().numpy(), r[k]), k
    for n in (1, 2, 63):
        g = tav.verify_tree_greedy(dev(draft[:, :n]), dev(target[:, :n]), dev(par[:, :n]))
        r = oracle.verify_greedy(draft[:, :n], target[:, :n], par[:, :n])
        assert np.array_equal(g["accepted_path"].cpu().numpy(), r["accepted_path"])


def test_chain_equals_causal():
    wl = W_["chain8"].with_(B=2, P=500)
    inp = gen.make_inputs(wl, 6, "cuda")
    g = gpu_masks(inp)
    out, lse = run_attention(inp, g["masks"])
    for b in range(wl.B):
        L = wl.P + wl.N
        pt = inp.page_table[b]
        kk = inp.k_cache[torch.as_tensor(pt.astype(np.int64)).cuda()]   # [pages][Hkv][ps][D]
        vv = inp.v_cache[torch.as_tensor(pt.astype(np.int64)).cuda()]
        kk = kk.permute(0, 2, 1, 3).reshape(-1, wl.Hkv, wl.D)[:L]
        vv = vv.permute(0, 2, 1, 3).reshape(-1, wl.Hkv, wl.D)[:L]
        co, cl = oracle.causal_attention(gen.bf16_bits(inp.q[b]), gen.bf16_bits(kk),
                                         gen.bf16_bits(vv))
        check_attention(out[b:b + 1], lse[b:b + 1], co, cl, tag="chain-vs-causal")


# ---------------------------------------------------------------------------
# full workload sizes, sampled rows
# ---------------------------------------------------------------------------

FULL = ["random16", "eagle64", "long64", "lanes", "chain8", "long64_fp8", "chain8_fp8",
        "long64_tp8"]


def group_rows(wl, b, g):
    """Flat (b * R + r) * Hq + h ids of every row of request b's kv head g:
    all rows one prefix workgroup folds, over every split of the prefix."""
    G = wl.Hq // wl.Hkv
    return np.array([(b * wl.R + r) * wl.Hq + h for r in range(wl.R)
                     for h in range(g * G, (g + 1) * G)], np.int64)


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    wl = W_[name]
    say("full", name, wl)
    inp = gen.make_inputs(wl, 1000 + FULL.index(name), "cuda")
    if wl.tree == "lanes":
        m_np = inp.lane_masks
        m_dev = dev(m_np.view(np.int64), torch.int64)
    else:
        g = gpu_masks(inp)
        r = oracle.build_masks(inp.parents, vc=inp.prefix_len)
        assert np.array_equal(masks_np(g["masks"]), r["masks"])
        assert np.array_equal(g["positions"].cpu().numpy(), r["positions"])
        m_dev, m_np = g["masks"], r["masks"]
        gv = tav.verify_tree_greedy(dev(inp.draft), dev(inp.target), dev(inp.parents))
        rv = oracle.verify_greedy(inp.draft, inp.target, inp.parents)
        for k in ("accepted_path", "accept_len", "accepted_tokens"):
            assert np.array_equal(gv[k].cpu().numpy(), rv[k]), k
    out, lse = run_attention(inp, m_dev)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    n_rows = wl.B * wl.R * wl.Hq
    rng = np.random.default_rng(7)
    # every row of the last request's last kv head, plus rows sampled anywhere
    rows = np.unique(np.concatenate([[0, n_rows - 1], rng.integers(0, n_rows, 40),
                                     group_rows(wl, wl.B - 1, wl.Hkv - 1)]))
    ro, rl = oracle_attention(inp, m_np, rows=rows)
    check_attention(out, lse, ro, rl, rows=rows, tag="full-%s (%d rows)" % (name, rows.size))
