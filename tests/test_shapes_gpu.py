"""GPU parity over seeded random shapes: tree_attention and the MLA cascade
through the C ABI against the CPU fp64 oracle, every row, with the bars of
the other parity tests (out max |err| <= 1e-2, lse2 max |err| <= 1e-3), and
the integer steps of a verify round (masks, greedy walk, compaction, shift)
bit-exact.

Each case draws its shape from its own seed: head dim 64 or 128, bf16 or FP8
E4M3 caches, 1 to 8 kv heads with 1 to 16 query heads each, 1 to 64 tree
rows (so every prefix kernel shape and row-group count comes up), pages of
1 to 256 keys, HND or NHD pools, ragged prefixes that include empty ones,
and sliding prefix windows.  The sizes keep the oracle under a few seconds
per case.
"""
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
    print("[shapes]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tav.lib()


def dev(x, dtype=torch.int32):
    return torch.as_tensor(np.ascontiguousarray(x)).to(dtype).cuda()


def compare(o, l, ro, rl, tag):
    o = o.reshape(-1, o.shape[-1])
    l = l.reshape(-1)
    ro = ro.reshape(o.shape)
    rl = rl.reshape(l.shape)
    assert np.isfinite(o).all(), tag + ": non-finite output"
    err = float(np.abs(o - ro).max())
    both_inf = np.isneginf(l) & np.isneginf(rl)
    lerr = float(np.abs(np.where(both_inf, 0.0, l - rl)).max())
    say(tag, "max|out err| %.2e  max|lse2 err| %.2e" % (err, lerr))
    assert err <= OUT_TOL and lerr <= LSE_TOL, (tag, err, lerr)


def attention_case(k):
    r = np.random.default_rng(7000 + k)
    D = int(r.choice([64, 128]))
    kv = str(r.choice(["", "fp8"]))
    Hkv = int(r.choice([1, 2, 4, 8]))
    G = int(r.choice([1, 2, 4, 8, 16]))
    N = int(r.integers(1, 65))
    B = int(r.integers(1, 5))
    ps = int(r.choice([1, 2, 4, 8, 16, 32, 64, 256]))
    rows = B * N * Hkv * G
    P = int(max(1, min(3000, 4_000_000 // (rows * D // 64 + 1))))
    P = int(r.integers(max(1, P // 3), P + 1))
    pl = r.integers(0, P + 1, B)
    pl[r.integers(0, B)] = P                       # one request at the full length
    if B > 1 and r.random() < 0.5:
        pl[r.integers(0, B)] = 0                   # and sometimes an empty prefix
    window = int(r.integers(1, P + 1)) if r.random() < 0.3 else 0
    layout = "NHD" if r.random() < 0.3 else "HND"
    tree = "chain" if r.random() < 0.2 else "random"
    wl = gen.Workload("shape%d" % k, B, P, N, Hkv * G, Hkv, D, "bf16", ps, tree,
                      depth_cap=int(r.integers(1, 9)), prefix_window=window, kv_dtype=kv)
    return wl, pl.astype(np.int32), layout


@pytest.mark.parametrize("k", range(24))
def test_random_shape_attention(k):
    wl, pl, layout = attention_case(k)
    tag = "case %d: B %d N %d Hq %d Hkv %d D %d %s ps %d P %s window %d %s" % (
        k, wl.B, wl.N, wl.Hq, wl.Hkv, wl.D, wl.kv, wl.page_size, pl.tolist(), wl.prefix_window,
        layout)
    say(tag)
    inp = gen.make_inputs(wl, 300 + k, "cuda", layout=layout, prefix_lens=pl)
    m = oracle.build_masks(inp.parents)["masks"]
    out, lse = tav.tree_attention(inp.q, inp.k_cache, inp.v_cache, dev(inp.page_table),
                                  dev(inp.prefix_len), dev(m.view(np.int64), torch.int64), wl.W,
                                  max_prefix_len=int(pl.max()), layout=layout,
                                  prefix_window=wl.prefix_window)
    torch.cuda.synchronize()
    ro, rl = oracle.tree_attention(gen.bf16_bits(inp.q), gen.bf16_bits(inp.k_cache),
                                   gen.bf16_bits(inp.v_cache), inp.strides, inp.page_table,
                                   wl.page_size, inp.prefix_len, m, wl.W, wl.Hkv,
                                   prefix_window=wl.prefix_window)
    compare(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, tag)


def mla_case(k):
    r = np.random.default_rng(8000 + k)
    Dr = int(r.choice([0, 64]))
    Hq = int(r.integers(1, 41))
    N = int(r.integers(1, 33))
    B = int(r.integers(1, 4))
    ps = int(r.choice([1, 4, 16, 64, 128]))
    rows = B * N * Hq
    P = int(max(1, min(2500, 1_500_000 // (rows * 9 + 1))))
    P = int(r.integers(max(1, P // 3), P + 1))
    pl = r.integers(0, P + 1, B)
    pl[r.integers(0, B)] = P
    kv = str(r.choice(["", "fp8"]))
    wl = gen.MlaWorkload("mshape%d" % k, B, P, N, Hq, 512, Dr, ps,
                         depth_cap=int(r.integers(1, 7)), kv_dtype=kv)
    return wl, pl.astype(np.int32)


@pytest.mark.parametrize("k", range(8))
def test_random_shape_mla(k):
    wl, pl = mla_case(k)
    tag = "mla case %d: B %d N %d Hq %d Dr %d %s ps %d P %s" % (
        k, wl.B, wl.N, wl.Hq, wl.Dr, wl.kv, wl.page_size, pl.tolist())
    say(tag)
    inp = gen.make_mla_inputs(wl, 400 + k, "cuda", prefix_lens=pl)
    m = oracle.build_masks(inp.parents)["masks"]
    out, lse = tav.tree_attention_mla(inp.q, inp.latent, dev(inp.page_table), dev(inp.prefix_len),
                                      dev(m.view(np.int64), torch.int64), wl.W, Dc=wl.Dc,
                                      max_prefix_len=int(pl.max()))
    torch.cuda.synchronize()
    ro, rl = oracle.mla_attention(gen.bf16_bits(inp.q), gen.bf16_bits(inp.latent), inp.strides,
                                  inp.page_table, wl.page_size, inp.prefix_len, m, wl.W, wl.Dc,
                                  wl.Dr)
    compare(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, tag)


def as_bytes(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16).numpy().view(np.uint8) if t.dtype == torch.bfloat16 \
        else t.view(torch.uint8).numpy()


def step_case(k):
    r = np.random.default_rng(9000 + k)
    B = int(r.integers(1, 17))
    N = int(r.integers(1, 65))
    D = int(r.choice([64, 128]))
    dtype, kv = [("bf16", ""), ("f32", ""), ("bf16", "fp8")][int(r.integers(0, 3))]
    Hkv = int(r.choice([1, 2, 8]))
    ps = int(r.choice([1, 4, 16, 64]))
    P = int(r.integers(0, 400))
    pl = r.integers(0, P + 1, B).astype(np.int32)
    tree = "chain" if r.random() < 0.25 else "random"
    layout = "NHD" if r.random() < 0.4 else "HND"
    wl = gen.Workload("step%d" % k, B, P, N, Hkv, Hkv, D, dtype, ps, tree,
                      depth_cap=int(r.integers(1, 10)), kv_dtype=kv)
    hidden_words = int(r.integers(1, 200))
    return wl, pl, layout, hidden_words


@pytest.mark.parametrize("k", range(12))
def test_random_shape_verify_step(k):
    """Masks, depth and positions; the greedy walk; compaction of the K and V
    caches and a hidden-state table; the position shift: bit-exact against
    the oracle on a random shape (1-16 requests, 1-64 nodes, pages of 1-64
    keys, HND or NHD pools of bf16, fp32 or FP8 rows, hidden rows of 1-199
    words)."""
    wl, pl, layout, hw = step_case(k)
    tag = "step case %d: B %d N %d D %d %s/%s Hkv %d ps %d P %s %s %s hidden %d" % (
        k, wl.B, wl.N, wl.D, wl.dtype, wl.kv, wl.Hkv, wl.page_size, pl.tolist(), layout,
        wl.tree, hw)
    say(tag)
    inp = gen.make_inputs(wl, 500 + k, "cuda", layout=layout, prefix_lens=pl)
    g = tav.tree_build_masks(dev(inp.parents), vc=dev(inp.prefix_len))
    ref = oracle.build_masks(inp.parents, vc=inp.prefix_len)
    torch.cuda.synchronize()
    assert np.array_equal(g["masks"].cpu().numpy().view(np.uint64), ref["masks"]), tag
    for key in ("depth", "positions", "tree_error"):
        assert np.array_equal(g[key].cpu().numpy(), ref[key]), (tag, key)
    v = tav.verify_tree_greedy(dev(inp.draft), dev(inp.target), dev(inp.parents))
    rv = oracle.verify_greedy(inp.draft, inp.target, inp.parents)
    for key in ("accepted_path", "accept_len", "accepted_tokens"):
        assert np.array_equal(v[key].cpu().numpy(), rv[key]), (tag, key)
    hidden = torch.randint(-2**31, 2**31 - 1, (wl.B, wl.N, hw), dtype=torch.int32, device="cuda")
    pt, pld = dev(inp.page_table), dev(inp.prefix_len)
    tables = [tav.RowTable.paged_kv(inp.k_cache, pt, pld, layout),
              tav.RowTable.paged_kv(inp.v_cache, pt, pld, layout),
              tav.RowTable.dense_rows(hidden)]
    host = []
    for t in tables:
        paged = t.page_table is not None
        host.append(dict(buf=as_bytes(t.buf).copy(), page_table=inp.page_table if paged else None,
                         prefix_len=inp.prefix_len if paged else None, page_size=t.page_size,
                         stride_page=t.stride_page, stride_token=t.stride_token,
                         stride_head=t.stride_head, stride_batch=t.stride_batch,
                         n_heads=t.n_heads, row_bytes=t.row_bytes))
    tav.compact_window_rows(tables, v["accepted_path"], v["accept_len"])
    torch.cuda.synchronize()
    oracle.compact_rows(host, rv["accepted_path"], rv["accept_len"])
    for name, t, h in zip(("K", "V", "hidden"), tables, host):
        assert np.array_equal(as_bytes(t.buf), h["buf"]), (tag, name)
    chain = inp.prefix_len[:, None] + np.arange(wl.N, dtype=np.int32)[None]
    p = dev(chain)
    tav.tree_shift_positions(p, g["depth"], +1)
    torch.cuda.synchronize()
    assert np.array_equal(p.cpu().numpy(), oracle.shift_positions(chain, ref["depth"], +1)), tag
    tav.tree_shift_positions(p, g["depth"], -1)
    torch.cuda.synchronize()
    assert np.array_equal(p.cpu().numpy(), chain), tag
