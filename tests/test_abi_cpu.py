"""The C-ABI library on the host: it loads, exports every function the header
declares, computes the static plan from (K, split_k) alone, and rejects bad
arguments with the documented status before any HIP call.  No test here
launches a kernel: every call below carries at least one defect that the host
checks catch (or is an M == 0 no-op), so fake device addresses are never
dereferenced."""
import ctypes
import os
import re

import pytest

import deterministic_split_lora_amd as dsl
from deterministic_split_lora_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora_det.h")

FAKE = 0x100000          # a 16-byte aligned address that is never dereferenced
FAKE_MIS = 0x100002      # misaligned


def header_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_function():
    L = dsl.lib()
    declared = header_functions()
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(L, name), f"{name} declared in lora_det.h but not exported"
    assert sorted(B.EXPORTED) == declared


def test_abi_version_and_status_strings():
    assert dsl.lora_abi_version() == 6
    seen = set()
    for s in range(0, 8):
        t = dsl.lora_status_str(s)
        assert t and t != "unknown status"
        seen.add(t)
    assert len(seen) == 8
    assert dsl.lora_status_str(99) == "unknown status"


@pytest.mark.parametrize("K,S,chunk,waves,steps", [
    (1024, 8, 128, 4, 1),      # single-adapter shrink, 8 tokens x 1024, 128-wide chunks
    (4096, 8, 512, 8, 2),      # q_proj-shaped 4096 hidden
    (14336, 8, 1792, 8, 7),    # MLP down-projection shape
    (8192, 16, 512, 8, 2),     # 8192 hidden, Split-K 16
    (8192, 8, 1024, 8, 4),
    (3072, 8, 384, 4, 3),      # the paper's decode example (hidden 3072)
    (4096, 1, 4096, 8, 16),
    (64, 2, 32, 1, 1),
])
def test_static_plan(K, S, chunk, waves, steps):
    p = dsl.lora_shrink_plan(K, 16, S)
    assert p == {"split_k": S, "k_chunk": chunk, "waves": waves, "k_steps": steps,
                 "rank_tiles": 1, "row_block": 16}
    assert waves * steps * 32 == chunk and chunk * S == K
    for r, rt in [(1, 1), (8, 1), (16, 1), (17, 2), (32, 2), (33, 3), (64, 4), (65, 5), (96, 6), (128, 8)]:
        assert dsl.lora_shrink_plan(K, r, S)["rank_tiles"] == rt


def test_plan_rejects():
    L = dsl.lib()
    p = B.ShrinkPlan()
    assert L.lora_shrink_plan(4096, 16, 3, ctypes.byref(p)) == B.LORA_ERR_UNSUPPORTED
    assert L.lora_shrink_plan(4096, 16, 32, ctypes.byref(p)) == B.LORA_ERR_UNSUPPORTED
    assert L.lora_shrink_plan(4096, 0, 8, ctypes.byref(p)) == B.LORA_ERR_UNSUPPORTED
    assert L.lora_shrink_plan(4096, 129, 8, ctypes.byref(p)) == B.LORA_ERR_UNSUPPORTED
    assert L.lora_shrink_plan(4000, 16, 8, ctypes.byref(p)) == B.LORA_ERR_UNSUPPORTED
    assert L.lora_shrink_plan(0, 16, 8, ctypes.byref(p)) == B.LORA_ERR_SHAPE
    assert L.lora_shrink_plan(4096, 16, 8, None) == B.LORA_ERR_NULL


def test_workspace_and_plan_sizes():
    assert dsl.lora_shrink_workspace_bytes(256, 16, 8) == 8 * 256 * 16 * 4
    assert dsl.lora_shrink_workspace_bytes(256, 16, 1) == 0
    assert dsl.lora_shrink_workspace_bytes(-1, 16, 8) == 0
    assert dsl.lora_shrink_workspace_bytes(256, 0, 8) == 0
    assert dsl.lora_shrink_workspace_bytes(256, 16, 3) == 0
    assert dsl.lora_sgmv_workspace_bytes(512, 64, 8) == 8 * 512 * 64 * 4
    assert dsl.lora_sgmv_workspace_bytes(512, 64, 1) == 512 * 64 * 4
    assert dsl.lora_sgmv_plan_bytes(512) == 16 + 16 * 512
    assert dsl.lora_sgmv_plan_bytes(-3) == 0


def _shrink(**kw):
    a = dict(x=FAKE, ld_x=4096, A=FAKE, ld_a=4096, h=FAKE, ld_h=16, M=4, K=4096, r=16, S=8, scale=1.0,
             ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return dsl.lib().lora_shrink_splitk(a["x"], a["ld_x"], a["A"], a["ld_a"], a["h"], a["ld_h"], a["M"], a["K"],
                                        a["r"], a["S"], a["scale"], a["ws"], a["wsb"], a["stream"])


def _atomic(**kw):
    a = dict(x=FAKE, ld_x=4096, A=FAKE, ld_a=4096, h=FAKE, ld_h=16, M=4, K=4096, r=16, S=8, scale=1.0)
    a.update(kw)
    return dsl.lib().lora_shrink_splitk_atomic(a["x"], a["ld_x"], a["A"], a["ld_a"], a["h"], a["ld_h"], a["M"],
                                               a["K"], a["r"], a["S"], a["scale"], None)


def _expand(fn="lora_expand", **kw):
    a = dict(h=FAKE, ld_h=16, B=FAKE, ld_b=16, y=FAKE, ld_y=4096, M=4, r=16, N=4096, scale=2.0)
    a.update(kw)
    return getattr(dsl.lib(), fn)(a["h"], a["ld_h"], a["B"], a["ld_b"], a["y"], a["ld_y"], a["M"], a["r"], a["N"],
                                  a["scale"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), B.LORA_ERR_NULL),
    (dict(A=None), B.LORA_ERR_NULL),
    (dict(h=None), B.LORA_ERR_NULL),
    (dict(ws=None), B.LORA_ERR_NULL),
    (dict(M=-1), B.LORA_ERR_SHAPE),
    (dict(r=0), B.LORA_ERR_UNSUPPORTED),
    (dict(r=129), B.LORA_ERR_UNSUPPORTED),
    (dict(S=3), B.LORA_ERR_UNSUPPORTED),
    (dict(S=32), B.LORA_ERR_UNSUPPORTED),
    (dict(K=4000, ld_x=4000, ld_a=4000), B.LORA_ERR_UNSUPPORTED),
    (dict(K=0), B.LORA_ERR_SHAPE),
    (dict(ld_x=4088), B.LORA_ERR_SHAPE),
    (dict(ld_a=4000), B.LORA_ERR_SHAPE),
    (dict(ld_h=8), B.LORA_ERR_SHAPE),
    (dict(x=FAKE_MIS), B.LORA_ERR_ALIGN),
    (dict(A=FAKE_MIS), B.LORA_ERR_ALIGN),
    (dict(h=FAKE + 2), B.LORA_ERR_ALIGN),
    (dict(ws=FAKE + 8), B.LORA_ERR_ALIGN),
    (dict(ld_x=4100), B.LORA_ERR_ALIGN),
    (dict(ld_a=4100), B.LORA_ERR_ALIGN),
    (dict(wsb=8 * 4 * 16 * 4 - 1), B.LORA_ERR_WORKSPACE),
])
def test_shrink_rejects(kw, status):
    assert _shrink(**kw) == status


def test_shrink_zero_rows_is_noop():
    # M == 0 succeeds without touching any pointer (and without a GPU)
    assert _shrink(M=0, x=None, A=None, h=None, ws=None) == B.LORA_OK
    assert _atomic(M=0, x=None, A=None, h=None) == B.LORA_OK
    assert _expand(M=0, h=None, B=None, y=None) == B.LORA_OK
    assert _expand(N=0, h=None, B=None, y=None) == B.LORA_OK
    assert _expand(fn="lora_expand_compensated", M=0, h=None, B=None, y=None) == B.LORA_OK


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), B.LORA_ERR_NULL),
    (dict(S=5), B.LORA_ERR_UNSUPPORTED),
    (dict(r=200), B.LORA_ERR_UNSUPPORTED),
    (dict(ld_a=8), B.LORA_ERR_SHAPE),
    (dict(A=FAKE_MIS), B.LORA_ERR_ALIGN),
])
def test_atomic_rejects(kw, status):
    assert _atomic(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(h=None), B.LORA_ERR_NULL),
    (dict(B=None), B.LORA_ERR_NULL),
    (dict(y=None), B.LORA_ERR_NULL),
    (dict(M=-2), B.LORA_ERR_SHAPE),
    (dict(r=0), B.LORA_ERR_UNSUPPORTED),
    (dict(r=129), B.LORA_ERR_UNSUPPORTED),
    (dict(N=4092, ld_y=4096), B.LORA_ERR_UNSUPPORTED),
    (dict(ld_y=4088), B.LORA_ERR_SHAPE),
    (dict(ld_b=8), B.LORA_ERR_SHAPE),
    (dict(ld_b=20), B.LORA_ERR_ALIGN),
    (dict(y=FAKE_MIS), B.LORA_ERR_ALIGN),
    (dict(h=FAKE + 8), B.LORA_ERR_ALIGN),
    (dict(M=(1 << 31) - 1, N=(1 << 31) - 8, ld_y=(1 << 31)), B.LORA_ERR_SHAPE),
])
def test_expand_rejects(kw, status):
    assert _expand(**kw) == status
    assert _expand(fn="lora_expand_compensated", **kw) == status


def test_sgmv_rejects():
    L = dsl.lib()
    pb = dsl.lora_sgmv_plan_bytes(64)
    # plan
    assert L.lora_sgmv_plan(FAKE, 64, 4, None, pb, None) == B.LORA_ERR_NULL
    assert L.lora_sgmv_plan(None, 64, 4, FAKE, pb, None) == B.LORA_ERR_NULL
    assert L.lora_sgmv_plan(FAKE, 64, 0, FAKE, pb, None) == B.LORA_ERR_SHAPE
    assert L.lora_sgmv_plan(FAKE, 64, 4, FAKE, pb - 1, None) == B.LORA_ERR_WORKSPACE
    assert L.lora_sgmv_plan(FAKE, 64, 4, FAKE + 4, pb, None) == B.LORA_ERR_ALIGN
    assert L.lora_sgmv_plan(FAKE, -1, 4, FAKE, pb, None) == B.LORA_ERR_SHAPE
    wsb = dsl.lora_sgmv_workspace_bytes(64, 64, 8)

    def shrink(**kw):
        a = dict(x=FAKE, ld_x=4096, Ap=FAKE, ld_a=4096, ranks=FAKE, scales=None, ids=FAKE, n=4, plan=FAKE,
                 pb=pb, h=FAKE, ld_h=64, M=64, K=4096, r_max=64, S=8, ws=FAKE, wsb=wsb)
        a.update(kw)
        return L.lora_sgmv_shrink(a["x"], a["ld_x"], a["Ap"], a["ld_a"], a["ranks"], a["scales"], a["ids"], a["n"],
                                  a["plan"], a["pb"], a["h"], a["ld_h"], a["M"], a["K"], a["r_max"], a["S"],
                                  a["ws"], a["wsb"], None)
    assert shrink(Ap=None) == B.LORA_ERR_NULL
    assert shrink(ranks=None) == B.LORA_ERR_NULL
    assert shrink(ids=None) == B.LORA_ERR_NULL
    assert shrink(n=0) == B.LORA_ERR_SHAPE
    assert shrink(r_max=129) == B.LORA_ERR_UNSUPPORTED
    assert shrink(S=6) == B.LORA_ERR_UNSUPPORTED
    assert shrink(ld_h=32) == B.LORA_ERR_SHAPE
    assert shrink(ld_a=4092) == B.LORA_ERR_SHAPE
    assert shrink(ld_a=4100) == B.LORA_ERR_ALIGN
    assert shrink(wsb=wsb - 4) == B.LORA_ERR_WORKSPACE
    assert shrink(pb=pb - 4) == B.LORA_ERR_WORKSPACE
    assert shrink(M=0, x=None) == B.LORA_OK

    def expand(**kw):
        a = dict(h=FAKE, ld_h=64, Bp=FAKE, ranks=FAKE, scales=None, ids=FAKE, n=4, y=FAKE, ld_y=4096,
                 M=64, N=4096, r_max=64)
        a.update(kw)
        return L.lora_sgmv_expand(a["h"], a["ld_h"], a["Bp"], a["ranks"], a["scales"], a["ids"], a["n"],
                                  a["y"], a["ld_y"], a["M"], a["N"], a["r_max"], None)
    assert expand(Bp=None) == B.LORA_ERR_NULL
    assert expand(ids=None) == B.LORA_ERR_NULL
    assert expand(ranks=None) == B.LORA_ERR_NULL
    assert expand(n=0) == B.LORA_ERR_SHAPE
    assert expand(ld_h=60) == B.LORA_ERR_SHAPE
    assert expand(h=FAKE + 4) == B.LORA_ERR_ALIGN
    assert expand(N=4090) == B.LORA_ERR_UNSUPPORTED
    assert expand(r_max=0) == B.LORA_ERR_UNSUPPORTED
    assert expand(ld_y=2048) == B.LORA_ERR_SHAPE
    assert expand(y=FAKE_MIS) == B.LORA_ERR_ALIGN
    assert expand(M=0, h=None) == B.LORA_OK


def test_shrink_expand_rejects():
    L = dsl.lib()
    wsb = dsl.lora_shrink_expand_workspace_bytes(4, 16, 8)
    assert wsb == 8 * 4 * 16 * 4
    assert dsl.lora_shrink_expand_workspace_bytes(4, 16, 1) == 4 * 16 * 4

    def call(**kw):
        a = dict(x=FAKE, ld_x=4096, A=FAKE, ld_a=4096, B=FAKE, ld_b=16, h=FAKE, ld_h=16, y=FAKE, ld_y=4096, M=4,
                 K=4096, r=16, N=4096, S=8, ss=1.0, es=2.0, ws=FAKE, wsb=wsb)
        a.update(kw)
        return L.lora_shrink_expand(a["x"], a["ld_x"], a["A"], a["ld_a"], a["B"], a["ld_b"], a["h"], a["ld_h"],
                                    a["y"], a["ld_y"], a["M"], a["K"], a["r"], a["N"], a["S"], a["ss"], a["es"],
                                    a["ws"], a["wsb"], None)
    assert call(x=None) == B.LORA_ERR_NULL
    assert call(B=None) == B.LORA_ERR_NULL
    assert call(y=None) == B.LORA_ERR_NULL
    assert call(ws=None) == B.LORA_ERR_NULL
    assert call(S=3) == B.LORA_ERR_UNSUPPORTED
    assert call(r=0) == B.LORA_ERR_UNSUPPORTED
    assert call(N=4090) == B.LORA_ERR_UNSUPPORTED
    assert call(K=4000, ld_x=4000, ld_a=4000) == B.LORA_ERR_UNSUPPORTED
    assert call(ld_b=8) == B.LORA_ERR_SHAPE
    assert call(ld_h=8) == B.LORA_ERR_SHAPE
    assert call(h=None, ld_h=8, ld_y=100) == B.LORA_ERR_SHAPE
    assert call(M=-1) == B.LORA_ERR_SHAPE
    assert call(y=FAKE_MIS) == B.LORA_ERR_ALIGN
    assert call(h=FAKE + 2) == B.LORA_ERR_ALIGN
    assert call(ld_b=20) == B.LORA_ERR_ALIGN
    assert call(wsb=wsb - 1) == B.LORA_ERR_WORKSPACE
    assert call(M=0, x=None, ws=None) == B.LORA_OK


def test_partials_and_combine_reject():
    L = dsl.lib()
    wsb = dsl.lora_shrink_expand_workspace_bytes(4, 16, 8)
    assert L.lora_shrink_partials(None, 4096, FAKE, 4096, 4, 4096, 16, 8, FAKE, wsb, None) == B.LORA_ERR_NULL
    assert L.lora_shrink_partials(FAKE, 4096, FAKE, 4096, 4, 4096, 16, 8, None, wsb, None) == B.LORA_ERR_NULL
    assert L.lora_shrink_partials(FAKE, 4096, FAKE, 4096, 4, 4096, 16, 6, FAKE, wsb, None) == B.LORA_ERR_UNSUPPORTED
    assert L.lora_shrink_partials(FAKE, 4096, FAKE, 4096, 4, 4096, 16, 8, FAKE, wsb - 4, None) == B.LORA_ERR_WORKSPACE
    assert L.lora_shrink_partials(FAKE_MIS, 4096, FAKE, 4096, 4, 4096, 16, 8, FAKE, wsb, None) == B.LORA_ERR_ALIGN
    assert L.lora_shrink_partials(FAKE, 2048, FAKE, 4096, 4, 4096, 16, 8, FAKE, wsb, None) == B.LORA_ERR_SHAPE
    assert L.lora_shrink_partials(None, 4096, None, 4096, 0, 4096, 16, 8, None, 0, None) == B.LORA_OK

    def comb(**kw):
        a = dict(ws=FAKE, wsb=wsb, S=8, ss=1.0, B=FAKE, ld_b=16, h=None, ld_h=0, y=FAKE, ld_y=4096, M=4, r=16,
                 N=4096, es=2.0)
        a.update(kw)
        return L.lora_expand_combine(a["ws"], a["wsb"], a["S"], a["ss"], a["B"], a["ld_b"], a["h"], a["ld_h"],
                                     a["y"], a["ld_y"], a["M"], a["r"], a["N"], a["es"], None)
    assert comb(ws=None) == B.LORA_ERR_NULL
    assert comb(B=None) == B.LORA_ERR_NULL
    assert comb(S=12) == B.LORA_ERR_UNSUPPORTED
    assert comb(r=129) == B.LORA_ERR_UNSUPPORTED
    assert comb(N=12) == B.LORA_ERR_UNSUPPORTED
    assert comb(wsb=wsb - 1) == B.LORA_ERR_WORKSPACE
    assert comb(h=FAKE, ld_h=8) == B.LORA_ERR_SHAPE
    assert comb(ld_y=8) == B.LORA_ERR_SHAPE
    assert comb(ws=FAKE + 4) == B.LORA_ERR_ALIGN
    assert comb(h=FAKE + 1, ld_h=16) == B.LORA_ERR_ALIGN
    assert comb(M=0, ws=None, B=None, y=None) == B.LORA_OK


def test_shrink_expand_fused_rejects():
    L = dsl.lib()

    def call(**kw):
        a = dict(x=FAKE, ld_x=4096, A=FAKE, ld_a=4096, B=FAKE, ld_b=16, h=FAKE, ld_h=16, y=FAKE, ld_y=4096, M=4,
                 K=4096, r=16, N=4096, S=8, ss=1.0, es=2.0)
        a.update(kw)
        return L.lora_shrink_expand_fused(a["x"], a["ld_x"], a["A"], a["ld_a"], a["B"], a["ld_b"], a["h"],
                                          a["ld_h"], a["y"], a["ld_y"], a["M"], a["K"], a["r"], a["N"], a["S"],
                                          a["ss"], a["es"], None)
    assert call(x=None) == B.LORA_ERR_NULL
    assert call(A=None) == B.LORA_ERR_NULL
    assert call(S=32) == B.LORA_ERR_UNSUPPORTED
    assert call(r=70) == B.LORA_ERR_UNSUPPORTED
    assert call(N=100, ld_y=4096) == B.LORA_ERR_UNSUPPORTED
    assert call(ld_x=2048) == B.LORA_ERR_SHAPE
    assert call(x=FAKE_MIS) == B.LORA_ERR_ALIGN
    assert call(h=FAKE + 1) == B.LORA_ERR_ALIGN
    assert call(M=0, x=None, A=None) == B.LORA_OK


def test_shrink_expand_launch_count():
    assert dsl.lora_shrink_expand_launches(1, 1024, 8, 4096, 8) == 1
    assert dsl.lora_shrink_expand_launches(64, 1024, 16, 4096, 8) == 1
    assert dsl.lora_shrink_expand_launches(65, 1024, 16, 4096, 8) == 2
    assert dsl.lora_shrink_expand_launches(1, 4096, 16, 4096, 8) == 2
    assert dsl.lora_shrink_expand_launches(0, 4096, 16, 4096, 8) == 0
    # the tree in a kernel of its own: many column blocks x splits, or many h values per column block
    assert dsl.lora_shrink_expand_launches(300, 2048, 64, 8200, 16) == 3
    assert dsl.lora_shrink_expand_launches(2100, 1024, 64, 1032, 8) == 3
    assert dsl.lora_shrink_expand_launches(1024, 14336, 32, 4096, 8) == 2
    assert dsl.lora_shrink_expand_launches(2048, 14336, 32, 4096, 8) == 3
    assert dsl.lora_shrink_expand_launches(8, 4000, 16, 4096, 8) < 0


def test_counted_rejects():
    L = dsl.lib()
    # one int32 per 16-wide rank tile of a rank <= 128, per row block / per plan tile
    assert dsl.lora_shrink_counter_bytes(1) == 32
    assert dsl.lora_shrink_counter_bytes(33) == 96
    assert dsl.lora_sgmv_counter_bytes(33) == 1056
    # tagged 64-bit slots: twice the two-pass workspace
    wsb = dsl.lora_counted_workspace_bytes(4, 16, 8)
    assert wsb == 2 * dsl.lora_shrink_workspace_bytes(4, 16, 8)

    def call(**kw):
        a = dict(x=FAKE, ld_x=4096, A=FAKE, ld_a=4096, h=FAKE, ld_h=16, M=4, K=4096, r=16, S=8, scale=1.0,
                 ws=FAKE, wsb=wsb, cnt=FAKE, cb=32)
        a.update(kw)
        return L.lora_shrink_splitk_counted(a["x"], a["ld_x"], a["A"], a["ld_a"], a["h"], a["ld_h"], a["M"],
                                            a["K"], a["r"], a["S"], a["scale"], a["ws"], a["wsb"], a["cnt"], a["cb"],
                                            None)
    assert call(cnt=None) == B.LORA_ERR_NULL
    assert call(ws=None) == B.LORA_ERR_NULL
    assert call(cnt=FAKE + 2) == B.LORA_ERR_ALIGN
    assert call(cb=0) == B.LORA_ERR_WORKSPACE
    assert call(wsb=wsb - 4) == B.LORA_ERR_WORKSPACE
    assert call(wsb=dsl.lora_shrink_workspace_bytes(4, 16, 8)) == B.LORA_ERR_WORKSPACE
    assert call(S=5) == B.LORA_ERR_UNSUPPORTED
    assert call(M=0, x=None, cnt=None) == B.LORA_OK
    pb = dsl.lora_sgmv_plan_bytes(64)
    wsg = dsl.lora_counted_workspace_bytes(64, 64, 8)

    def sg(**kw):
        a = dict(x=FAKE, ld_x=4096, Ap=FAKE, ld_a=4096, ranks=FAKE, scales=None, n=4, plan=FAKE, pb=pb, h=FAKE,
                 ld_h=64, M=64, K=4096, r_max=64, S=8, ws=FAKE, wsb=wsg, cnt=FAKE, cb=1024)
        a.update(kw)
        return L.lora_sgmv_shrink_counted(a["x"], a["ld_x"], a["Ap"], a["ld_a"], a["ranks"], a["scales"], a["n"],
                                          a["plan"], a["pb"], a["h"], a["ld_h"], a["M"], a["K"], a["r_max"], a["S"],
                                          a["ws"], a["wsb"], a["cnt"], a["cb"], None)
    assert sg(cnt=None) == B.LORA_ERR_NULL
    assert sg(plan=None) == B.LORA_ERR_NULL
    assert sg(cb=1020) == B.LORA_ERR_WORKSPACE
    assert sg(wsb=dsl.lora_sgmv_workspace_bytes(64, 64, 8)) == B.LORA_ERR_WORKSPACE
    assert sg(n=0) == B.LORA_ERR_SHAPE
    assert sg(cnt=FAKE + 1) == B.LORA_ERR_ALIGN
    assert sg(M=0, x=None) == B.LORA_OK


def test_shrink_expand_counted_rejects():
    L = dsl.lib()
    assert dsl.lora_shrink_expand_counter_bytes(1) == 16 + 8
    assert dsl.lora_shrink_expand_counter_bytes(33) == 16 + 3 * 8
    assert dsl.lora_shrink_expand_counter_bytes(0) == 16
    assert dsl.lora_shrink_expand_counter_bytes(-1) == 0
    wsb = dsl.lora_shrink_expand_workspace_bytes(4, 16, 8)
    cbytes = dsl.lora_shrink_expand_counter_bytes(4)

    def call(**kw):
        a = dict(x=FAKE, ld_x=4096, A=FAKE, ld_a=4096, B=FAKE, ld_b=16, h=FAKE, ld_h=16, y=FAKE, ld_y=4096, M=4,
                 K=4096, r=16, N=4096, S=8, ss=1.0, es=2.0, ws=FAKE, wsb=wsb, cnt=FAKE, cb=cbytes)
        a.update(kw)
        return L.lora_shrink_expand_counted(a["x"], a["ld_x"], a["A"], a["ld_a"], a["B"], a["ld_b"], a["h"],
                                            a["ld_h"], a["y"], a["ld_y"], a["M"], a["K"], a["r"], a["N"], a["S"],
                                            a["ss"], a["es"], a["ws"], a["wsb"], a["cnt"], a["cb"], None)
    assert call(x=None) == B.LORA_ERR_NULL
    assert call(B=None) == B.LORA_ERR_NULL
    assert call(ws=None) == B.LORA_ERR_NULL
    assert call(cnt=None) == B.LORA_ERR_NULL
    assert call(S=3) == B.LORA_ERR_UNSUPPORTED
    assert call(r=129) == B.LORA_ERR_UNSUPPORTED
    assert call(N=4092) == B.LORA_ERR_UNSUPPORTED
    assert call(ld_h=8) == B.LORA_ERR_SHAPE
    assert call(M=-5) == B.LORA_ERR_SHAPE
    assert call(y=FAKE_MIS) == B.LORA_ERR_ALIGN
    assert call(ws=FAKE + 8) == B.LORA_ERR_ALIGN
    assert call(cnt=FAKE + 2) == B.LORA_ERR_ALIGN
    assert call(wsb=wsb - 4) == B.LORA_ERR_WORKSPACE
    assert call(cb=cbytes - 1) == B.LORA_ERR_WORKSPACE
    assert call(M=0, x=None, ws=None, cnt=None) == B.LORA_OK
    assert call(N=0, ws=None, cnt=None) == B.LORA_OK


def test_sgmv_shrink_expand_rejects():
    L = dsl.lib()
    pb = dsl.lora_sgmv_plan_bytes(64)
    wsb = dsl.lora_sgmv_workspace_bytes(64, 64, 8)

    def call(**kw):
        a = dict(x=FAKE, ld_x=4096, Ap=FAKE, ld_a=4096, Bp=FAKE, ranks=FAKE, ss=None, es=None, ids=FAKE, n=4,
                 plan=FAKE, pb=pb, h=None, ld_h=0, y=FAKE, ld_y=6144, M=64, K=4096, N=6144, r_max=64, S=8, ws=FAKE,
                 wsb=wsb)
        a.update(kw)
        return L.lora_sgmv_shrink_expand(a["x"], a["ld_x"], a["Ap"], a["ld_a"], a["Bp"], a["ranks"], a["ss"], a["es"],
                                         a["ids"], a["n"], a["plan"], a["pb"], a["h"], a["ld_h"], a["y"], a["ld_y"],
                                         a["M"], a["K"], a["N"], a["r_max"], a["S"], a["ws"], a["wsb"], None)
    assert call(x=None) == B.LORA_ERR_NULL
    assert call(Bp=None) == B.LORA_ERR_NULL
    assert call(ids=None) == B.LORA_ERR_NULL
    assert call(ws=None) == B.LORA_ERR_NULL
    assert call(n=0) == B.LORA_ERR_SHAPE
    assert call(S=3) == B.LORA_ERR_UNSUPPORTED
    assert call(r_max=129) == B.LORA_ERR_UNSUPPORTED
    assert call(N=6140, ld_y=6144) == B.LORA_ERR_UNSUPPORTED
    assert call(ld_y=4096) == B.LORA_ERR_SHAPE
    assert call(h=FAKE, ld_h=32) == B.LORA_ERR_SHAPE
    assert call(h=FAKE + 2, ld_h=64) == B.LORA_ERR_ALIGN
    assert call(y=FAKE_MIS) == B.LORA_ERR_ALIGN
    assert call(pb=pb - 4) == B.LORA_ERR_WORKSPACE
    assert call(wsb=wsb - 4) == B.LORA_ERR_WORKSPACE
    assert call(wsb=dsl.lora_shrink_workspace_bytes(4, 16, 8)) == B.LORA_ERR_WORKSPACE
    assert call(M=0, x=None, ws=None) == B.LORA_OK


def test_noalloc_rejects_sizes_beyond_its_scratch_buffer():
    """split_k * M * r * 4 above the fixed 8 MiB buffer is refused on the host,
    before any pointer is looked at or any HIP call is made; the limit itself
    passes the size check (and then fails on the NULL pointers)."""
    L = dsl.lib()
    assert B.NOALLOC_SCRATCH_BYTES == 8 << 20
    args = lambda M, r, S: (None, 4096, None, 4096, None, 64, None, 0, None, 4096, M, 4096, r, 4096, S,
                            ctypes.c_float(1.0), ctypes.c_float(2.0), None)
    # 8 * 4096 * 64 * 4 = 8 MiB: fits; one more token does not
    assert L.lora_shrink_expand_noalloc(*args(4096, 64, 8)) == B.LORA_ERR_NULL
    assert L.lora_shrink_expand_noalloc(*args(4097, 64, 8)) == B.LORA_ERR_SCRATCH
    assert L.lora_shrink_expand_noalloc(*args(1 << 20, 16, 16)) == B.LORA_ERR_SCRATCH
    # the usual shape and plan checks come first
    assert L.lora_shrink_expand_noalloc(*args(-1, 16, 8)) == B.LORA_ERR_SHAPE
    assert L.lora_shrink_expand_noalloc(*args(16, 16, 3)) == B.LORA_ERR_UNSUPPORTED
    assert L.lora_shrink_expand_noalloc(*args(0, 16, 8)) == B.LORA_OK
