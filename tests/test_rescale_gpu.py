"""GPU parity of the prefix kernels' softmax-reference changes.

Both MFMA prefix kernels avoid a per-block rescale of their partial output:
the small-row-group kernel raises its running maximum only when a 32-key
block beats it by more than 8 (log2 units), and the wide-row-group kernel
keeps the maximum of its first block as the reference and moves it only when
the running sum of weights would pass 2^20 or a weight overflows.  N(0, 1)
inputs never reach those branches, so these cases plant scores that do:

  sawtooth   channel 0 of every prefix key rises by ~40 log2 units over each
             256-key period (the running maximum is raised every few blocks;
             the wide kernel's weight sum passes 2^20 within a period)
  staircase  +14 log2 units every 96 keys, four steps then back to 0 (blocks
             that beat the running maximum by 8-20: 0 < alpha < 1)
  spike      a key every 700 scoring ~200 log2 units above the rest (its
             weight relative to the first block is infinite in fp32)

Every query row gets channel 0 = 8, so the planted key channel moves every
row's score by about the same amount (8 * k0 * log2(e) / sqrt(128) ~ k0 log2
units).  Each case runs for every prefix kernel shape (32, 64, 128 and 256
folded rows per kv head) in bf16 and with FP8 E4M3 caches, with ragged
prefixes and with a sliding window whose first key is not 8-aligned (the
split's first 32-key block then starts with keys that are not visible).
Every row is compared with the CPU fp64 oracle: out max |err| <= 1e-2, lse2
max |err| <= 1e-3.
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
    print("[rescale]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tav.lib()


def dev(x, dtype=torch.int32):
    return torch.as_tensor(np.ascontiguousarray(x)).to(dtype).cuda()


def key_channel0(pattern, t):
    """Planted value of channel 0 of prefix key t (numpy int array)."""
    if pattern == "sawtooth":
        return 40.0 * (t % 256) / 256.0
    if pattern == "staircase":
        return 14.0 * ((t // 96) % 5)
    if pattern == "spike":
        return np.where(t % 700 == 650, 200.0, 0.0)
    raise ValueError(pattern)


def plant(inp, pattern):
    """q channel 0 = 8 everywhere; channel 0 of every visible prefix key of
    every kv head = the pattern (window keys keep their N(0, 1) values)."""
    wl = inp.wl
    inp.q[..., 0] = 8.0
    ps = wl.page_size
    for b in range(wl.B):
        P = int(inp.prefix_len[b])
        if P == 0:
            continue
        t = np.arange(P)
        pages = torch.as_tensor(inp.page_table[b, t // ps].astype(np.int64), device="cuda")
        slots = torch.as_tensor((t % ps).astype(np.int64), device="cuda")
        vals = torch.as_tensor(key_channel0(pattern, t), dtype=torch.float32, device="cuda")
        vals = vals.to(inp.k_cache.dtype)
        kc = inp.k_cache
        if kc.dtype == torch.float8_e4m3fn:      # write the E4M3 bytes
            kc, vals = kc.view(torch.uint8), vals.view(torch.uint8)
        for g in range(wl.Hkv):
            if inp.layout == "HND":
                kc[pages, g, slots, 0] = vals
            else:
                kc[pages, slots, g, 0] = vals


# (R, Hq, Hkv): R * Hq / Hkv folded rows per kv head -> the kernel shape
SHAPES = {"rows32": (8, 8, 2), "rows64": (16, 8, 2), "rows128": (32, 8, 2),
          "rows256": (64, 8, 2)}


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("shape", sorted(SHAPES))
@pytest.mark.parametrize("pattern", ["sawtooth", "staircase", "spike"])
@pytest.mark.parametrize("window", [0, 1000])
def test_reference_changes(pattern, shape, kv, window):
    R, Hq, Hkv = SHAPES[shape]
    # window 1000 over prefixes of 3003 / 2411: the visible range starts at
    # 2003 / 1411, not on an 8-key boundary
    pl = [3003, 2411] if window else [3000, 2047]
    wl = gen.Workload("rescale", 2, max(pl), R, Hq, Hkv, 128, "bf16", 16, "random",
                      depth_cap=6, prefix_window=window, kv_dtype="" if kv == "bf16" else kv)
    seed = 40 + 7 * sorted(SHAPES).index(shape) + (3 if window else 0)
    inp = gen.make_inputs(wl, seed, "cuda", prefix_lens=pl)
    plant(inp, pattern)
    m = oracle.build_masks(inp.parents)["masks"]
    out, lse = tav.tree_attention(inp.q, inp.k_cache, inp.v_cache, dev(inp.page_table),
                                  dev(inp.prefix_len), dev(m.view(np.int64), torch.int64), wl.W,
                                  max_prefix_len=max(pl), prefix_window=window)
    torch.cuda.synchronize()
    ro, rl = oracle.tree_attention(gen.bf16_bits(inp.q), gen.bf16_bits(inp.k_cache),
                                   gen.bf16_bits(inp.v_cache), inp.strides, inp.page_table,
                                   wl.page_size, inp.prefix_len, m, wl.W, wl.Hkv,
                                   prefix_window=window)
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(l).all()
    err = float(np.abs(o - ro.reshape(o.shape)).max())
    lerr = float(np.abs(l - rl.reshape(l.shape)).max())
    # the planted scores must dominate: lse2 far above the N(0, 1) level
    assert float(np.median(rl)) > 20.0
    say("%s %s %s window %d: max|out err| %.2e  max|lse2 err| %.2e  median lse2 %.1f"
        % (pattern, shape, kv, window, err, lerr, float(np.median(rl))))
    assert err <= OUT_TOL
    assert lerr <= LSE_TOL
