"""A whole verify step captured in a HIP graph and replayed.

Every call of the path writes only buffers its caller bound before, launches
on the caller's stream, allocates nothing and never synchronises with the
host, so a serving loop can capture a step once and replay it (the drafter of
"EAGLE-style speculative decoding ... worked iteration" replays a captured
multi-step graph; "Draft-tree speculation", section "Draft lanes write the
draft cache like any draft step", keeps its buffers at fixed addresses for
that reason).  This test captures the six calls of one step (masks, prefix,
window + merge, greedy walk, compaction of K, V and a hidden-state table,
position shift) through the C ABI, replays the graph three times with the
caches restored eagerly in between, and compares every output and every
byte of the compacted tables with an eager run of the same calls: bit for
bit.
"""
import sys

import numpy as np
import pytest
import torch

import tree_attention_verify_amd as tav
from tree_attention_verify_amd import inputs as gen

pytestmark = pytest.mark.gpu


def say(*a):
    print("[graph]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tav.lib()


class Step:
    """Buffers bound once and the six C calls of one verify step."""

    def __init__(self, wl, inp):
        self.wl, self.inp = wl, inp
        t = lambda x, dt=torch.int32: torch.as_tensor(np.ascontiguousarray(x)).to(dt).cuda()
        B, N, R = wl.B, wl.N, wl.R
        self.parents, self.prefix_len = t(inp.parents), t(inp.prefix_len)
        self.page_table = t(inp.page_table)
        self.draft, self.target = t(inp.draft), t(inp.target)
        e = lambda shape, dt=torch.int32: torch.empty(shape, dtype=dt, device="cuda")
        self.depth, self.masks, self.positions = e((B, N)), e((B, N), torch.int64), e((B, N))
        self.tree_error = e((B,))
        self.out = torch.empty_like(inp.q)
        self.lse = e((B, R, wl.Hq), torch.float32)
        self.path, self.alen, self.tokens = e((B, N)), e((B,)), e((B, N))
        g = torch.Generator(device="cuda")
        g.manual_seed(123)
        self.hidden = torch.randn((B, N, 512), device="cuda", generator=g).to(torch.bfloat16)
        sp, sh, st, Hkv, ps = tav.kv_strides(inp.k_cache, inp.layout)
        self.kv = (sp, sh, st, inp.k_cache.shape[0], ps)
        self.code = tav._code(inp.q.dtype, inp.k_cache.dtype)
        nb = tav.tree_attention_workspace_size(inp.q.dtype, B, R, wl.Hq, wl.Hkv, wl.D,
                                               int(inp.prefix_len.max()), wl.prefix_window, ps,
                                               inp.k_cache.dtype)
        self.ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        tabs = [tav.RowTable.paged_kv(inp.k_cache, self.page_table, self.prefix_len),
                tav.RowTable.paged_kv(inp.v_cache, self.page_table, self.prefix_len),
                tav.RowTable.dense_rows(self.hidden)]
        self.tables = (tav.TavRows * 3)()
        for i, tb in enumerate(tabs):
            self.tables[i] = tav.TavRows(
                tb.buf.data_ptr(), None if tb.page_table is None else tb.page_table.data_ptr(),
                None if tb.prefix_len is None else tb.prefix_len.data_ptr(),
                0 if tb.page_table is None else tb.page_table.shape[1], tb.page_size,
                tb.num_pages, tb.stride_page, tb.stride_token, tb.stride_head, tb.stride_batch,
                tb.n_heads, tb.row_bytes)
        # the caches and the hidden table as they were before any step
        self.saved = [inp.k_cache.clone(), inp.v_cache.clone(), self.hidden.clone()]

    def restore(self):
        for dst, src in zip((self.inp.k_cache, self.inp.v_cache, self.hidden), self.saved):
            dst.copy_(src)

    def run(self):
        L, wl, inp = tav.lib(), self.wl, self.inp
        B, N = wl.B, wl.N
        s = torch.cuda.current_stream().cuda_stream
        chk = lambda rc: tav._check(rc)
        chk(L.tree_build_masks(self.parents.data_ptr(), B, N, self.prefix_len.data_ptr(),
                               self.depth.data_ptr(), self.masks.data_ptr(),
                               self.positions.data_ptr(), self.tree_error.data_ptr(), s))
        sp, sh, st, npages, ps = self.kv
        for fn in (L.tree_attention_prefix, L.tree_attention_window_merge):
            chk(fn(inp.q.data_ptr(), inp.k_cache.data_ptr(), inp.v_cache.data_ptr(), self.code,
                   sp, sh, st, npages, self.page_table.data_ptr(), self.page_table.shape[1], ps,
                   self.prefix_len.data_ptr(), int(inp.prefix_len.max()), wl.prefix_window,
                   self.masks.data_ptr(), wl.W, B, wl.R, wl.Hq, wl.Hkv, wl.D, 0.0,
                   self.out.data_ptr(), self.lse.data_ptr(), self.ws.data_ptr(), self.ws.numel(),
                   s))
        chk(L.verify_tree_greedy(self.draft.data_ptr(), self.target.data_ptr(),
                                 self.parents.data_ptr(), B, N, self.path.data_ptr(),
                                 self.alen.data_ptr(), self.tokens.data_ptr(), s))
        chk(L.compact_window_rows(self.tables, 3, self.path.data_ptr(), self.alen.data_ptr(), B,
                                  N, s))
        chk(L.tree_shift_positions(self.positions.data_ptr(), self.depth.data_ptr(), B, N, -1,
                                   s))

    def snapshot(self):
        raw = lambda x: x.detach().contiguous().view(torch.uint8).cpu().numpy().copy()
        return {"depth": raw(self.depth), "masks": raw(self.masks),
                "positions": raw(self.positions), "tree_error": raw(self.tree_error),
                "out": raw(self.out), "lse2": raw(self.lse), "path": raw(self.path),
                "accept_len": raw(self.alen), "tokens": raw(self.tokens),
                "k_cache": raw(self.inp.k_cache), "v_cache": raw(self.inp.v_cache),
                "hidden": raw(self.hidden)}


CASES = {
    # 256 folded rows (the pipelined prefix kernel), several splits
    "long64": gen.WORKLOADS["long64"].with_(B=2, P=3000),
    # 64 folded rows, page size 16
    "random16": gen.WORKLOADS["random16"].with_(B=3, P=1000),
    # FP8 E4M3 caches
    "chain8_fp8": gen.WORKLOADS["chain8_fp8"].with_(B=4, P=2000),
    # 512 folded rows in one split: the prefix phase takes the window keys and
    # writes the output, the window-and-merge phase launches nothing
    "eagle64": gen.WORKLOADS["eagle64"].with_(B=2, P=300),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_captured_step_replays_bit_exact(name):
    wl = CASES[name]
    say("case", name, wl)
    inp = gen.make_inputs(wl, 31, "cuda")
    step = Step(wl, inp)
    step.run()
    torch.cuda.synchronize()
    eager = step.snapshot()
    # the step really moved rows: some request accepted more than the root
    assert int(step.alen.max()) > 1 or wl.tree == "chain"

    step.restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):      # warm the capture stream first
        step.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    step.restore()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step.run()
    torch.cuda.synchronize()
    for rep in range(3):
        step.restore()
        for x in (step.out, step.lse, step.path, step.masks, step.positions):
            x.zero_()                 # replays must rewrite every output
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = step.snapshot()
        for k in eager:
            assert np.array_equal(got[k], eager[k]), "replay %d: %s differs" % (rep, k)
    say(name, "three replays bit-identical to the eager step")
