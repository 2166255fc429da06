"""tree_attention_noalloc (partials in the library's fixed device array)
against tree_attention (partials in a caller workspace): two calls in a row
on one GPU, the second smaller than the first, each compared with
tree_attention on the same inputs (same kernels, so bit for bit) and with
the CPU fp64 oracle on sampled rows (out max |err| <= 1e-2, lse2 max |err|
<= 1e-3).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verify_amd as tav
from tree_attention_verify_amd import inputs as gen

pytestmark = pytest.mark.gpu


def say(*a):
    print("[noalloc]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tav.lib()


def dev(x, dtype=torch.int32):
    return torch.as_tensor(np.ascontiguousarray(x)).to(dtype).cuda()


def one_call(wl, seed, prefix_lens=None):
    inp = gen.make_inputs(wl, seed, "cuda", prefix_lens=prefix_lens)
    m = oracle.build_masks(inp.parents)["masks"]
    md = dev(m.view(np.int64), torch.int64)
    pt, pl = dev(inp.page_table), dev(inp.prefix_len)
    P = int(inp.prefix_len.max())
    need = tav.tree_attention_workspace_size(inp.q.dtype, wl.B, wl.R, wl.Hq, wl.Hkv, wl.D, P,
                                             wl.prefix_window, wl.page_size, inp.k_cache.dtype)
    assert need <= tav.NOALLOC_SCRATCH_BYTES
    ref_o, ref_l = tav.tree_attention(inp.q, inp.k_cache, inp.v_cache, pt, pl, md, wl.W,
                                      max_prefix_len=P, prefix_window=wl.prefix_window)
    out = torch.full_like(inp.q, float("nan"))
    lse = torch.full((wl.B, wl.R, wl.Hq), float("nan"), dtype=torch.float32, device="cuda")
    tav.tree_attention_noalloc(inp.q, inp.k_cache, inp.v_cache, pt, pl, md, wl.W,
                               max_prefix_len=P, out=out, lse2=lse,
                               prefix_window=wl.prefix_window)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                       ref_o.view(torch.int16) if ref_o.dtype == torch.bfloat16 else ref_o)
    assert torch.equal(lse, ref_l)
    n_rows = wl.B * wl.R * wl.Hq
    rows = np.unique(np.concatenate([[0, n_rows - 1],
                                     np.random.default_rng(seed).integers(0, n_rows, 64)]))
    ro, rl = oracle.tree_attention(gen.bf16_bits(inp.q), gen.bf16_bits(inp.k_cache),
                                   gen.bf16_bits(inp.v_cache), inp.strides, inp.page_table,
                                   wl.page_size, inp.prefix_len, m, wl.W, wl.Hkv,
                                   prefix_window=wl.prefix_window, rows=rows)
    o = out.float().cpu().numpy().reshape(n_rows, wl.D)[rows]
    l = lse.cpu().numpy().reshape(-1)[rows]
    err = float(np.abs(o - ro).max())
    lerr = float(np.abs(l - rl).max())
    say("%s: %d bytes of partials, bit-identical to tree_attention; vs oracle max|out err| "
        "%.2e max|lse2 err| %.2e" % (wl.describe(), need, err, lerr))
    assert err <= 1e-2 and lerr <= 1e-3


def test_noalloc_matches_tree_attention_twice():
    # the long-context workload at its full size (the largest partials the
    # fixed array is sized for), then a smaller ragged one
    one_call(gen.WORKLOADS["long64"], 71)
    one_call(gen.WORKLOADS["random16"].with_(B=3, P=1000), 72, prefix_lens=[1000, 37, 513])


def test_noalloc_fp8_and_small_rows():
    one_call(gen.WORKLOADS["chain8_fp8"].with_(B=4, P=2000), 73, prefix_lens=[2000, 1, 64, 1999])
    one_call(gen.WORKLOADS["worked"], 74)


def test_noalloc_one_split_window_in_prefix_launch():
    # 512 folded rows in one split: the prefix launch takes the window keys
    # and writes the output itself, for both entry points
    one_call(gen.WORKLOADS["eagle64"].with_(B=2, P=300), 75, prefix_lens=[300, 0])
