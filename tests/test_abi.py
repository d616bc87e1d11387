"""The C ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any HIP call (CPU only: no kernels run)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tree_attn.h")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"TA_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from tree_masked_attention_forward_amd import _binding
    return _binding.load_library()


def test_header_declares_the_three_calls():
    names = _declared_functions()
    for n in ("tree_attn_build_mask", "tree_attn_forward", "tree_verify_greedy",
              "tree_attn_mask_and_forward", "tree_kv_commit", "tree_verify_greedy_next",
              "tree_attn_forward_noalloc", "tree_verify_sample"):
        assert n in names
    assert len(names) == 12, names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_product_library_carries_no_timeline_code(lib):
    """The per-workgroup timestamps exist only in the timeline build
    (libtreeattn_timeline.so, a measurement tool); the library the package
    loads exports no timeline entry."""
    assert not hasattr(lib, "ta_timeline_set")


def test_timeline_summary_on_a_made_up_stamp_table():
    """bench.py's timeline summary (host arithmetic only) on stamps whose
    answers are known: 256 split workgroups with a 10 us loop over 8 tiles
    on 16 CUs, and 128 merge workgroups."""
    import importlib.util
    import sys

    import numpy as np
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    argv = sys.argv
    try:
        sys.argv = ["bench.py"]
        spec.loader.exec_module(bench)
    finally:
        sys.argv = argv
    n = 384
    t = np.zeros((n, 16), np.int64)
    t[:, 0] = 1000
    t[:, 1] = t[:, 0] + 100        # 1 us
    t[:, 2] = t[:, 1] + 300        # 4 us
    t[:, 3] = t[:, 2] + 1000       # 14 us: a 10 us loop
    t[:, 4] = t[:, 3] + 100
    t[:, 5] = t[:, 4] + 100        # 16 us
    t[:256, 6] = 1
    t[256:, 6] = 2
    t[:, 14] = 8
    t[:, 15] = (np.arange(n) % 16) << 8
    r = bench.timeline_summary(t)
    assert r["splits"] == 256 and r["merge_workgroups"] == 128
    assert r["span_us"] == 16.0
    assert r["split"]["loop_us_per_tile"]["p50"] == 1.25
    assert r["split"]["before_loop_us"]["p50"] == 4.0
    assert r["cus"]["used"] == 16
    assert r["cus"]["tiles_per_cu"]["p50"] == 16 * 8


def test_status_strings(lib):
    from tree_masked_attention_forward_amd import _binding as b
    for code in range(6):
        assert b.status_string(code)
    assert b.status_string(99) == "unknown status"


def _fwd(lib, **kw):
    args = dict(dtype=1, q=1 << 20, kt=1 << 20, vt=1 << 20, kp=1 << 20, vp=1 << 20, po=1 << 20,
                pl=None, no=1 << 20, mask=1 << 20, B=1, total=64, maxn=64, tp=4096, mp=4096, Hq=32,
                Hkv=8,
                D=128, scale=0.088, out=1 << 20, lse=None, ws=None, wsb=0, stream=None)
    args.update(kw)
    a = args
    return lib.tree_attn_forward(a["dtype"], a["q"], a["kt"], a["vt"], a["kp"], a["vp"], a["po"],
                                 a["pl"], a["no"], a["mask"], a["B"], a["total"], a["maxn"], a["tp"],
                                 a["mp"], a["Hq"], a["Hkv"], a["D"], a["scale"], a["out"],
                                 a["lse"], a["ws"], a["wsb"], a["stream"])


def test_forward_host_validation(lib):
    assert _fwd(lib, dtype=7) == 3                 # unknown dtype
    assert _fwd(lib, B=0) == 1
    assert _fwd(lib, Hq=30, Hkv=8) == 1            # Hq % Hkv != 0
    assert _fwd(lib, D=64) == 3                    # bf16 path needs D == 128
    assert _fwd(lib, dtype=0, D=300) == 3          # fp32 path: D <= 256
    assert _fwd(lib, maxn=5000) == 3               # above TA_MAX_NODES
    assert _fwd(lib, q=None) == 1
    assert _fwd(lib, kp=None) == 1                 # prefix rows but no prefix pointer
    assert _fwd(lib, q=(1 << 20) + 2) == 1         # misaligned bf16 pointer
    assert _fwd(lib, mp=5000) == 1                 # max_prefix > total_prefix
    assert _fwd(lib, scale=float("nan")) == 1
    assert _fwd(lib, ws=None, wsb=0) == 4          # this shape needs split partials
    assert _fwd(lib, total=0) == 0                 # nothing to do, nothing launched


def test_workspace_queries_are_pure_host(lib):
    from tree_masked_attention_forward_amd import _binding as b
    import torch
    n = b.forward_workspace_size(torch.bfloat16, 1, 64, 64, 32, 8, 128, 4096, 4096)
    assert n > 0 and n % 16 == 0
    assert b.forward_workspace_size(torch.float32, 1, 5, 5, 1, 1, 64, 16, 16) == 0
    assert b.verify_workspace_size(64, 64, 128256) >= 64 * 8
    assert b.verify_workspace_size(0, 1, 10) == 0
    # Up to 1024 nodes the workspace is the chunk results only (4 chunks of a
    # 128256-entry row, 8 bytes each); above, per-row scratch follows them
    # (prediction and depth 4 bytes, match word and key 8 bytes, each array
    # 256-byte aligned).
    small = b.verify_workspace_size(4096, 1024, 128256)
    assert small == 4096 * 4 * 8
    big = b.verify_workspace_size(4096, 4096, 128256)
    assert big == small + 2 * 4096 * 4 + 2 * 4096 * 8


def test_build_mask_and_verify_host_validation(lib):
    assert lib.tree_attn_build_mask(1 << 20, 1 << 20, 0, 5, 5, 1 << 20, None, None, None) == 1
    assert lib.tree_attn_build_mask(1 << 20, 1 << 20, 1, 5, 4097, 1 << 20, None, None, None) == 3
    assert lib.tree_attn_build_mask(None, 1 << 20, 1, 5, 5, 1 << 20, None, None, None) == 1
    v = lib.tree_verify_greedy
    ok = [1, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1, 64, 64, 1000, None, 1 << 20, 1 << 20,
          1 << 20, 1 << 20, 1 << 20, None]
    bad_dtype = list(ok); bad_dtype[0] = 5
    assert v(*bad_dtype) == 3
    no_ws = list(ok); no_ws[14] = 0
    assert v(*no_ws) == 4
    no_len = list(ok); no_len[10] = None
    assert v(*no_len) == 1
    big = list(ok); big[7] = 5000
    assert v(*big) == 3


def _mfwd(lib, **kw):
    args = dict(dtype=1, par=1 << 20, q=1 << 20, kt=1 << 20, vt=1 << 20, kp=1 << 20, vp=1 << 20,
                po=1 << 20, pl=None, no=1 << 20, B=1, total=64, maxn=64, tp=4096, mp=4096, Hq=32,
                Hkv=8, D=128, scale=0.088, mask=1 << 20, depth=None, status=None, out=1 << 20,
                lse=None,
                ws=None, wsb=0, stream=None)
    args.update(kw)
    a = args
    return lib.tree_attn_mask_and_forward(
        a["dtype"], a["par"], a["q"], a["kt"], a["vt"], a["kp"], a["vp"], a["po"], a["pl"], a["no"],
        a["B"], a["total"], a["maxn"], a["tp"], a["mp"], a["Hq"], a["Hkv"], a["D"], a["scale"],
        a["mask"], a["depth"], a["status"], a["out"], a["lse"], a["ws"], a["wsb"], a["stream"])


def test_mask_and_forward_host_validation(lib):
    assert _mfwd(lib, dtype=7) == 3
    assert _mfwd(lib, Hq=30, Hkv=8) == 1
    assert _mfwd(lib, maxn=5000) == 3
    assert _mfwd(lib, q=None) == 1
    assert _mfwd(lib, par=None) == 1               # parents are required
    assert _mfwd(lib, mask=None) == 1              # the mask is an output here
    assert _mfwd(lib, ws=None, wsb=0) == 4         # split partials need a workspace
    assert _mfwd(lib, maxn=200, ws=None, wsb=0) == 4   # two-call path checks it too
    assert _mfwd(lib, total=0) == 0                # nothing to do, nothing launched


def _commit(lib, **kw):
    args = dict(dtype=1, kt=1 << 20, vt=1 << 20, no=1 << 20, al=1 << 20, an=1 << 20, B=2,
                total=10, maxn=8, Hkv=8, D=128, kc=1 << 20, vc=1 << 20, co=1 << 20, cl=1 << 20,
                tc=100, st=None, stream=None)
    args.update(kw)
    a = args
    return lib.tree_kv_commit(a["dtype"], a["kt"], a["vt"], a["no"], a["al"], a["an"], a["B"],
                              a["total"], a["maxn"], a["Hkv"], a["D"], a["kc"], a["vc"], a["co"],
                              a["cl"], a["tc"], a["st"], a["stream"])


def test_kv_commit_host_validation(lib):
    assert _commit(lib, dtype=9) == 3
    assert _commit(lib, B=0) == 1
    assert _commit(lib, maxn=5000) == 3
    assert _commit(lib, Hkv=0) == 1
    assert _commit(lib, kt=None) == 1              # tree rows but no tree pointer
    assert _commit(lib, kc=None) == 1              # cache rows but no cache pointer
    assert _commit(lib, cl=None) == 1              # the lengths are required
    assert _commit(lib, tc=-1) == 1
    # A tree buffer inside a cache buffer is refused before any HIP call; each
    # case overlaps exactly one (tree, cache) pair.  (No case here passes the
    # checks: that would launch a kernel on made-up addresses.)
    row = 8 * 128 * 2
    far = dict(kt=1 << 30, vt=(1 << 30) + (1 << 24), kc=1 << 32, vc=(1 << 32) + (1 << 28))
    for tree, cache, at in (("kt", "kc", 0), ("vt", "vc", 99), ("kt", "vc", 50),
                            ("vt", "kc", -9)):
        kw = dict(far)
        kw[tree] = far[cache] + at * row   # 10 tree rows starting at cache row `at`
        assert _commit(lib, **kw) == 1, (tree, cache, at)


def test_verify_next_host_validation(lib):
    v = lib.tree_verify_greedy_next
    ok = [1, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 2, 64, 64, 1000, None, 1 << 20,
          1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, None]
    bad = list(ok); bad[0] = 5
    assert v(*bad) == 3
    bad = list(ok); bad[2] = None                  # the prefix rows are required
    assert v(*bad) == 1
    bad = list(ok); bad[14] = None                 # so is the bonus token
    assert v(*bad) == 1
    bad = list(ok); bad[16] = 8                    # workspace for sum_N + B rows
    assert v(*bad) == 4
    bad = list(ok); bad[8] = 5000
    assert v(*bad) == 3


def test_verify_sample_host_validation(lib):
    v = lib.tree_verify_sample
    #      dtype logits  root    q       q_root  draft   parents offsets B  N   maxn V
    ok = [1, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 2, 64, 64, 1000,
          #   T    u_acc    u_fin    alen     anodes   atok     bonus    ws       ws_bytes stream
          0.7, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 153408, None]
    bad = list(ok); bad[0] = 5
    assert v(*bad) == 3
    for i in (2, 4, 7, 14, 15, 16, 17, 18):        # always required
        bad = list(ok); bad[i] = None
        assert v(*bad) == 1, i
    for i in (1, 3, 5, 6, 13):                     # required when there are nodes
        bad = list(ok); bad[i] = None
        assert v(*bad) == 1, i
    for t in (0.0, -1.0, float("nan"), float("inf")):
        bad = list(ok); bad[12] = t
        assert v(*bad) == 1, t
    bad = list(ok); bad[20] = 153407                # rows and segment statistics
    assert v(*bad) == 4
    bad = list(ok); bad[19] = (1 << 20) + 8         # misaligned workspace
    assert v(*bad) == 4
    bad = list(ok); bad[10] = 5000
    assert v(*bad) == 3
    # two fp32 rows of V per sequence (256-byte aligned), then 260 float2 per row
    assert lib.tree_verify_sample_workspace_size(2, 64, 1000) == 16128 + 66 * 260 * 8
    assert lib.tree_verify_sample_workspace_size(0, 64, 1000) == 0


def _noalloc(lib, **kw):
    args = dict(dtype=1, q=1 << 20, kt=1 << 20, vt=1 << 20, kp=1 << 20, vp=1 << 20, po=1 << 20,
                pl=None, no=1 << 20, mask=1 << 20, B=1, total=64, maxn=64, tp=4096, mp=4096, Hq=32,
                Hkv=8, D=128, scale=0.088, out=1 << 20, lse=None, st=None, stream=None)
    args.update(kw)
    a = args
    return lib.tree_attn_forward_noalloc(a["dtype"], a["q"], a["kt"], a["vt"], a["kp"], a["vp"],
                                         a["po"], a["pl"], a["no"], a["mask"], a["B"], a["total"],
                                         a["maxn"], a["tp"], a["mp"], a["Hq"], a["Hkv"], a["D"],
                                         a["scale"], a["out"], a["lse"], a["st"], a["stream"])


def test_forward_noalloc_host_validation(lib):
    """The same host checks as tree_attn_forward, and a shape whose scratch
    exceeds the static array is refused before any HIP call."""
    assert _noalloc(lib, dtype=7) == 3
    assert _noalloc(lib, B=0) == 1
    assert _noalloc(lib, D=64) == 3
    assert _noalloc(lib, mask=None) == 1
    assert _noalloc(lib, total=0) == 0                 # nothing to do, nothing launched
    # 64 ragged sequences (262144 keys, the longest 65536) x 8 KV heads: each is cut into
    # key splits whose partials need far more than 64 MiB
    big = dict(B=64, total=64 * 64, tp=64 * 4096, mp=65536)
    need = lib.tree_attn_forward_workspace_size(1, big["B"], big["total"], 64, 32, 8, 128,
                                                big["tp"], big["mp"])
    assert need > 64 << 20, need
    assert _noalloc(lib, **big) == 4
