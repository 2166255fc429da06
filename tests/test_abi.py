"""C ABI checks that need no GPU: the library loads, exports every function
include/treeverify.h declares, and rejects bad arguments on the host with a
message naming every failed check, before anything is launched.

The rejected calls pass placeholder pointers, so they are only run where no
GPU is visible (a validation bug must never turn them into a launch).
"""
import ctypes
import os
import re

import pytest
import torch

import tree_attention_verify_amd as tav
from tree_attention_verify_amd import build as tav_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "treeverify.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tav.LIB_PATH):
        tav_build.build()
    return tav.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:tav_status|size_t|const char \*)\s*(\w+)\s*\(", text,
                                 flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("tree_build_masks", "tree_attention", "verify_tree_greedy", "compact_window_rows",
              "tree_shift_positions", "tree_attention_workspace_size"):
        assert n in names
    assert set(names) == set(tav.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), n
    assert L.tav_version().decode().startswith("treeverify")


def test_workspace_size_host_only(L):
    f = tav.tree_attention_workspace_size
    n = f(torch.bfloat16, 4, 64, 32, 8, 128, 131072, 0, 64)
    assert n > 0 and n % 256 == 0
    # fp32 partials: at least one (o, lse) per row
    assert n >= 4 * 64 * 32 * 129 * 4
    assert f(torch.bfloat16, 4, 65, 32, 8, 128, 1024, 0, 64) == 0      # R > 64
    assert f(torch.bfloat16, 4, 8, 30, 8, 128, 1024, 0, 64) == 0       # Hq % Hkv
    assert f(torch.bfloat16, 4, 8, 32, 8, 96, 1024, 0, 64) == 0        # D
    assert f(torch.bfloat16, 4, 8, 32, 8, 128, 1024, 0, 48) == 0       # page size
    assert f(torch.float32, 0, 8, 32, 8, 128, 0, 0, 16) > 0            # empty batch is fine


no_gpu = pytest.mark.skipif(torch.cuda.is_available(),
                            reason="placeholder pointers: run where no GPU is visible")
FAKE = 1 << 40  # 256-byte aligned placeholder, never dereferenced


def attn_call(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=tav.TAV_BF16, sp=8 * 64 * 128, sh=64 * 128, st=128,
             num_pages=100, pt=FAKE, max_pages=20, ps=64, plen=FAKE, maxp=1000, pw=0, masks=FAKE,
             W=64, B=2, R=64, Hq=32, Hkv=8, D=128, scale=0.0, out=FAKE, lse=FAKE, ws=FAKE,
             wsb=1 << 30)
    a.update(kw)
    st = L.tree_attention(a["q"], a["k"], a["v"], a["dtype"], a["sp"], a["sh"], a["st"],
                          a["num_pages"], a["pt"], a["max_pages"], a["ps"], a["plen"], a["maxp"],
                          a["pw"], a["masks"], a["W"], a["B"], a["R"], a["Hq"], a["Hkv"], a["D"],
                          a["scale"], a["out"], a["lse"], a["ws"], a["wsb"], None)
    return st, L.tav_last_error().decode()


@no_gpu
@pytest.mark.parametrize("kw,status,words", [
    (dict(R=65), 1, ["R must be in [1, 64]"]),
    (dict(W=65), 1, ["W must be in [0, 64]"]),
    (dict(Hq=30), 1, ["multiple of Hkv"]),
    (dict(D=96), 2, ["D must be 64 or 128"]),
    (dict(ps=48), 2, ["page_size"]),
    (dict(dtype=7), 2, ["dtype"]),
    (dict(max_pages=16), 1, ["must cover max_prefix_len + W"]),
    (dict(wsb=1024), 3, ["workspace has 1024 bytes"]),
    (dict(ws=FAKE + 16), 3, ["256-byte aligned"]),
    (dict(q=None), 1, ["q, k_cache and v_cache must be set"]),
    (dict(masks=None), 1, ["masks is NULL"]),
    (dict(st=100), 2, ["multiples of 16 bytes"]),
    (dict(scale=float("nan")), 1, ["sm_scale must be finite"]),
    (dict(B=-1), 1, ["B must be >= 0"]),
])
def test_tree_attention_rejects(L, kw, status, words):
    st, msg = attn_call(L, **kw)
    assert st == status, msg
    for w in words:
        assert w in msg, msg


@no_gpu
def test_tree_attention_reports_every_blocker(L):
    st, msg = attn_call(L, R=65, D=96, ps=48, W=70)
    assert st != 0
    for w in ("R must be", "D must be", "page_size", "W must be"):
        assert w in msg, msg


@no_gpu
def test_small_entry_points_reject(L):
    assert L.tree_build_masks(FAKE, 2, 65, None, FAKE, FAKE, None, None, None) == 1
    assert "N must be in [1, 64]" in L.tav_last_error().decode()
    assert L.tree_build_masks(None, 2, 8, None, FAKE, FAKE, None, None, None) == 1
    assert "parents is NULL" in L.tav_last_error().decode()
    assert L.tree_shift_positions(FAKE, FAKE, 2, 8, 0, None) == 1
    assert "direction" in L.tav_last_error().decode()
    assert L.verify_tree_greedy(FAKE, FAKE, FAKE, 2, 0, FAKE, FAKE, None, None) == 1
    assert L.verify_tree_greedy(FAKE, None, FAKE, 2, 8, FAKE, FAKE, None, None) == 1
    assert "target_argmax is NULL" in L.tav_last_error().decode()
    t = (tav.TavRows * 1)()
    t[0] = tav.TavRows(FAKE, None, None, 0, 1, 0, 0, 64, 0, 0, 1, 6)   # row_bytes % 4 != 0
    assert L.compact_window_rows(t, 1, FAKE, FAKE, 2, 8, None) == 1
    assert "row_bytes" in L.tav_last_error().decode()
    t[0] = tav.TavRows(FAKE, FAKE, None, 4, 16, 10, 0, 64, 0, 0, 1, 64)  # paged, no prefix_len
    assert L.compact_window_rows(t, 1, FAKE, FAKE, 2, 8, None) == 1
    assert "prefix_len is NULL" in L.tav_last_error().decode()


def noalloc_call(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=tav.TAV_BF16, sp=8 * 64 * 128, sh=64 * 128, st=128,
             num_pages=100, pt=FAKE, max_pages=20, ps=64, plen=FAKE, maxp=1000, pw=0, masks=FAKE,
             W=64, B=2, R=64, Hq=32, Hkv=8, D=128, scale=0.0, out=FAKE, lse=FAKE)
    a.update(kw)
    st = L.tree_attention_noalloc(a["q"], a["k"], a["v"], a["dtype"], a["sp"], a["sh"], a["st"],
                                  a["num_pages"], a["pt"], a["max_pages"], a["ps"], a["plen"],
                                  a["maxp"], a["pw"], a["masks"], a["W"], a["B"], a["R"], a["Hq"],
                                  a["Hkv"], a["D"], a["scale"], a["out"], a["lse"], None)
    return st, L.tav_last_error().decode()


@no_gpu
def test_noalloc_refuses_shapes_past_its_scratch(L):
    # B 32, R 64, Hq 64, Hkv 8, P 8192: ~135 MB of partials > 64 MiB
    st, msg = noalloc_call(L, B=32, Hq=64, maxp=8192, max_pages=8192 // 64 + 1)
    assert st == 3, msg
    assert "static scratch array" in msg and str(tav.NOALLOC_SCRATCH_BYTES) in msg, msg
    assert tav.tree_attention_workspace_size(torch.bfloat16, 32, 64, 64, 8, 128, 8192, 0, 64) \
        > tav.NOALLOC_SCRATCH_BYTES
    # argument errors are reported as for tree_attention
    st, msg = noalloc_call(L, R=65, D=96)
    assert st != 0 and "R must be" in msg and "D must be" in msg, msg


def test_noalloc_limit_matches_the_header():
    text = open(HEADER).read()
    assert re.search(r"#define TAV_NOALLOC_SCRATCH_BYTES \(\(size_t\)64 << 20\)", text)
    assert tav.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_empty_batch_is_a_no_op(L):
    # B = 0 launches nothing and succeeds (no pointer is touched)
    assert L.tree_build_masks(None, 0, 8, None, None, None, None, None, None) == 0
    assert L.verify_tree_greedy(None, None, None, 0, 8, None, None, None, None) == 0
    assert L.tree_shift_positions(None, None, 0, 8, 1, None) == 0
    st, msg = attn_call(L, B=0, q=None, k=None, v=None, pt=None, plen=None, masks=None,
                        out=None, lse=None, ws=None)
    assert st == 0, msg
    st, msg = noalloc_call(L, B=0, q=None, k=None, v=None, pt=None, plen=None, masks=None,
                           out=None, lse=None)
    assert st == 0, msg
    assert L.compact_window_rows(None, 0, None, None, 0, 8, None) == 0


def test_binding_refuses_cpu_tensors():
    with pytest.raises(ValueError):
        tav.tree_build_masks(torch.zeros((1, 4), dtype=torch.int32))


def test_sample_workspace_size_host_only(L):
    n = L.tree_sample_workspace_size(32, 64, 128256)
    assert n > 0 and n % 256 == 0
    assert L.tree_sample_workspace_size(32, 64, 128256) >= 32 * 64 * 8   # (z, token) per row
    assert L.tree_sample_workspace_size(-1, 64, 100) == 0
    assert L.tree_sample_workspace_size(2, 0, 100) == 0
    assert L.tree_sample_workspace_size(2, 8, 0) == 0


def sample_call(L, **kw):
    a = dict(logits=FAKE, dtype=tav.TAV_BF16, rs=128256, V=128256, B=2, N=8, T=FAKE, seed=FAKE,
             pos=FAKE, tok=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    st = L.tree_sample_gumbel(a["logits"], a["dtype"], a["rs"], a["V"], a["B"], a["N"], a["T"],
                              a["seed"], a["pos"], a["tok"], a["ws"], a["wsb"], None)
    return st, L.tav_last_error().decode()


@no_gpu
@pytest.mark.parametrize("kw,status,words", [
    (dict(N=65), 1, ["N must be in [1, 64]"]),
    (dict(V=0), 1, ["V must be >= 1"]),
    (dict(dtype=tav.TAV_FP8_E4M3), 2, ["logits dtype"]),
    (dict(rs=100), 1, ["row_stride must be >= V"]),
    (dict(rs=128260, V=128257), 1, ["multiple of 16 bytes"]),
    (dict(logits=FAKE + 8), 1, ["16-byte aligned"]),
    (dict(seed=None), 1, ["seed is NULL"]),
    (dict(pos=None), 1, ["positions is NULL"]),
    (dict(wsb=64), 3, ["workspace too small"]),
    (dict(ws=FAKE + 64), 3, ["256-byte aligned"]),
])
def test_tree_sample_gumbel_rejects(L, kw, status, words):
    st, msg = sample_call(L, **kw)
    assert st == status, msg
    for w in words:
        assert w in msg, msg


def test_sample_empty_batch_is_a_no_op(L):
    st, msg = sample_call(L, B=0, logits=None, T=None, seed=None, pos=None, tok=None, ws=None,
                          wsb=0)
    assert st == 0, msg


def rejection_call(L, **kw):
    a = dict(probs=FAKE, rs=128256, V=128256, q=None, qs=0, draft=FAKE, par=FAKE, score=None,
             coins=FAKE, bu=FAKE, B=4, N=64, path=FAKE, alen=FAKE, tok=FAKE, ws=FAKE,
             wsb=1 << 30)
    a.update(kw)
    st = L.verify_tree_rejection(a["probs"], a["rs"], a["V"], a["q"], a["qs"], a["draft"],
                                 a["par"], a["score"],
                                 a["coins"], a["bu"], a["B"], a["N"], a["path"], a["alen"],
                                 a["tok"], a["ws"], a["wsb"], None)
    return st, L.tav_last_error().decode()


@no_gpu
@pytest.mark.parametrize("kw,status,words", [
    (dict(N=0), 1, ["N must be in [1, 64]"]),
    (dict(V=(1 << 20) + 1, rs=(1 << 20) + 4), 1, ["V must be in [1, 1048576]"]),
    (dict(rs=1000), 1, ["row_stride must be >= V"]),
    (dict(rs=128258), 1, ["multiple of 4 elements"]),
    (dict(probs=FAKE + 4), 1, ["16-byte aligned"]),
    (dict(coins=None, bu=None), 1, ["coins is NULL", "bonus_u is NULL"]),
    (dict(path=None), 1, ["accepted_path is NULL"]),
    (dict(q=FAKE, qs=1000), 1, ["q_row_stride must be >= V"]),
    (dict(q=FAKE + 8, qs=128258), 1, ["multiple of 4 elements", "draft_q is not 16-byte aligned"]),
    (dict(ws=None), 3, ["workspace is NULL"]),
    (dict(ws=FAKE + 16), 3, ["workspace is not 256-byte aligned"]),
    (dict(wsb=1000), 3, ["workspace too small"]),
])
def test_verify_tree_rejection_rejects(L, kw, status, words):
    st, msg = rejection_call(L, **kw)
    assert st == status, msg
    for w in words:
        assert w in msg, msg


def test_rejection_empty_batch_is_a_no_op(L):
    st, msg = rejection_call(L, B=0, probs=None, draft=None, par=None, coins=None, bu=None,
                             path=None, alen=None, tok=None, ws=None, wsb=0)
    assert st == 0, msg


def test_rejection_workspace_size(L):
    f = L.verify_tree_rejection_workspace_size
    # out of range: 0
    assert f(-1, 64, 1000) == 0 and f(4, 0, 1000) == 0 and f(4, 65, 1000) == 0
    assert f(4, 64, 0) == 0 and f(4, 64, (1 << 20) + 1) == 0
    # grows with the batch and the vocabulary, in 256-byte units
    a, b, c = f(4, 64, 128256), f(32, 64, 128256), f(32, 64, 1 << 20)
    assert 0 < a < b < c and a % 256 == b % 256 == c % 256 == 0
    # at least the per-request tile sums of a row (one float per 256 tokens)
    assert b >= 32 * (128256 // 256) * 4


@no_gpu
def test_tree_construction_entry_points_reject(L):
    # beam step: the pool range and the candidate limit
    assert L.tree_beam_step(FAKE, FAKE, FAKE, FAKE, 2, 4, 4, 10, 0, FAKE, FAKE, FAKE, FAKE, FAKE,
                            None) == 1
    assert "pool_base" in L.tav_last_error().decode()
    assert L.tree_beam_step(FAKE, FAKE, FAKE, FAKE, 2, 64, 32, 5000, 0, FAKE, FAKE, FAKE, FAKE,
                            FAKE, None) == 2
    assert "<= 1024" in L.tav_last_error().decode()
    assert L.tree_beam_step(None, FAKE, FAKE, FAKE, 2, 4, 4, 100, 0, FAKE, FAKE, FAKE, FAKE, FAKE,
                            None) == 1
    # selection: N, C and order
    assert L.tree_select_candidates(FAKE, FAKE, FAKE, FAKE, 2, 100, 65, 0, FAKE, FAKE, FAKE, None,
                                    None) == 1
    assert "N must be in [1, 64]" in L.tav_last_error().decode()
    assert L.tree_select_candidates(FAKE, FAKE, FAKE, FAKE, 2, 5, 8, 0, FAKE, FAKE, FAKE, None,
                                    None) == 1
    assert "C must be >=" in L.tav_last_error().decode()
    assert L.tree_select_candidates(FAKE, FAKE, FAKE, FAKE, 2, 9000, 8, 0, FAKE, FAKE, FAKE, None,
                                    None) == 2
    assert L.tree_select_candidates(FAKE, FAKE, FAKE, FAKE, 2, 100, 8, 2, FAKE, FAKE, FAKE, None,
                                    None) == 1
    assert "order" in L.tav_last_error().decode()
    assert L.tree_retrieve_links(FAKE, 2, 0, FAKE, FAKE, None) == 1
    assert L.tree_retrieve_links(None, 2, 8, FAKE, FAKE, None) == 1
    # empty batches launch nothing
    assert L.tree_beam_step(None, None, None, None, 0, 4, 4, 100, 0, None, None, None, None, None,
                            None) == 0
    assert L.tree_select_candidates(None, None, None, None, 0, 100, 8, 1, None, None, None, None,
                                    None) == 0
    assert L.tree_retrieve_links(None, 0, 8, None, None, None) == 0


@no_gpu
def test_tree_attention_mla_rejects(L):
    def call(**kw):
        a = dict(q=FAKE, lat=FAKE, dtype=tav.TAV_BF16, sp=64 * 576, st=576, num_pages=100,
                 pt=FAKE, max_pages=20, ps=64, plen=FAKE, maxp=1000, masks=FAKE, W=16, B=2, R=16,
                 Hq=16, Dc=512, Dr=64, scale=0.0, out=FAKE, lse=FAKE, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        st = L.tree_attention_mla(a["q"], a["lat"], a["dtype"], a["sp"], a["st"], a["num_pages"],
                                  a["pt"], a["max_pages"], a["ps"], a["plen"], a["maxp"],
                                  a["masks"], a["W"], a["B"], a["R"], a["Hq"], a["Dc"], a["Dr"],
                                  a["scale"], a["out"], a["lse"], a["ws"], a["wsb"], None)
        return st, L.tav_last_error().decode()
    for kw, status, word in ((dict(Dc=256), 2, "Dc"), (dict(Dr=32), 2, "Dr must be 0 or 64"),
                             (dict(dtype=tav.TAV_F32), 2, "TAV_BF16"), (dict(R=65), 1, "R must be"),
                             (dict(max_pages=10), 1, "must cover"), (dict(st=100), 2, "16-byte"),
                             (dict(wsb=100), 3, "workspace has"), (dict(masks=None), 1, "masks")):
        st, msg = call(**kw)
        assert st == status and word in msg, (kw, st, msg)
    assert L.tree_attention_mla_workspace_size(2, 16, 16, 512, 64, 1000, 64) > 0
    assert L.tree_attention_mla_workspace_size(2, 16, 16, 256, 64, 1000, 64) == 0
    st, msg = call(B=0, q=None, lat=None, pt=None, plen=None, masks=None, out=None, lse=None,
                   ws=None)
    assert st == 0, msg


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus N > 1 exits with a message before
    touching a device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2, r.stderr[-500:]
    assert "one GPU" in r.stderr and r.stdout == ""
