"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, and rejects bad arguments on the host before launching
anything (so these calls never reach a HIP runtime call)."""
import ctypes
import os
import re

import numpy as np
import pytest

import attention_anchor_probe_amd as A
from attention_anchor_probe_amd import binding as Bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "acache.h")

FAKE = 0x10000          # 16-byte aligned non-null address: never dereferenced on these paths
FAKE_MIS = 0x10004      # misaligned


def declared():
    txt = open(HDR).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(acache_[a-z_]+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(Bd.LIB_PATH)
    names = declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(Bd.EXPORTS)


def test_version_and_status_strings():
    assert A.acache_version() >= 100
    lib = Bd._lib()
    for code in range(0, -10, -1):
        assert lib.acache_status_string(code) != b"unknown status"
    assert lib.acache_status_string(-99) == b"unknown status"


def test_anchor_count_matches_ceil_reading():
    assert A.acache_anchor_count(64, 0.2) == 13
    assert A.acache_anchor_count(1024, 0.2) == 205
    assert A.acache_anchor_count(4096, 0.2) == 820
    assert A.acache_anchor_count(16384, 0.3) == 4916
    assert A.acache_anchor_count(30, 0.1) == 3
    assert A.acache_anchor_count(5, 0.0) == 0 and A.acache_anchor_count(5, 1.0) == 5
    for bad in (-0.1, 1.01, float("nan")):
        with pytest.raises(A.AcacheError):
            A.acache_anchor_count(10, bad)


def pool(**kw):
    base = dict(k=FAKE, v=FAKE, dtype=1, n_layers=2, n_pages=8, page_size=16, n_kv_heads=2, head_dim=128)
    base.update(kw)
    return Bd.KVPool(**base)


def probe(p, **kw):
    a = dict(q=FAKE, n_rows=10, masked_rows=FAKE, masked_offsets=FAKE, n_masked=4, max_masked=4, shared_slots=FAKE,
             L=32, B=1, n_q_heads=4, layer_begin=0, n_layers=2, scale=0.088, scores=FAKE, o_aff=None, lse_aff=None,
             ws=FAKE * 16, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return Bd._lib().acache_probe_scores(ctypes.byref(p), a["q"], a["n_rows"], a["masked_rows"], a["masked_offsets"],
                                         a["n_masked"], a["max_masked"], a["shared_slots"], a["L"], a["B"],
                                         a["n_q_heads"], a["layer_begin"], a["n_layers"], a["scale"], a["scores"],
                                         a["o_aff"], a["lse_aff"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(), None),
    (dict(k=None), -1), (dict(dtype=5), -2), (dict(head_dim=96), -3), (dict(page_size=12), -3),
    (dict(page_size=512), -3), (dict(n_kv_heads=0), -3), (dict(k=FAKE_MIS), -9),
])
def test_probe_pool_validation(kw, code):
    st = probe(pool(**kw), B=0)    # B = 0: a valid call enqueues nothing
    assert st == (0 if code is None else code)


@pytest.mark.parametrize("kw,code", [
    (dict(n_q_heads=3), -3), (dict(layer_begin=1), -1), (dict(n_layers=3), -1), (dict(scale=0.0), -1),
    (dict(scale=float("inf")), -1), (dict(L=0), -1), (dict(max_masked=5), -1), (dict(shared_slots=None), -1),
    (dict(scores=None), -1), (dict(q=FAKE_MIS), -9), (dict(ws_bytes=16), -7), (dict(ws=None), -7),
    (dict(ws=FAKE + 16), -7),
])
def test_probe_argument_validation(kw, code):
    assert probe(pool(), **kw) == code


def test_probe_workspace_query():
    need = A.acache_probe_workspace_bytes(100, 3, 50, 4, 2, False)
    assert need >= 2 * 100 * 4 * 4 + 2 * 3 * 50 * 4
    assert A.acache_probe_workspace_bytes(100, 3, 50, 4, 2, True) < need


def test_topk_and_maps_validation():
    lib = Bd._lib()
    assert lib.acache_topk_anchors(FAKE, 1, 10, 11, 0, FAKE, None, None) == -1      # K > L
    assert lib.acache_topk_anchors(FAKE, 1, 10, -1, 0, FAKE, None, None) == -1
    assert lib.acache_topk_anchors(FAKE, 1, 40000, 5, 0, FAKE, None, None) == -3    # L above the select limit
    assert lib.acache_topk_anchors(None, 1, 10, 5, 0, FAKE, None, None) == -1
    m = Bd.MapArgs(1, 0, 10, 3, 16, 20, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    m_bad = Bd.MapArgs(1, 0, 10, 4, 16, 20, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    assert lib.acache_topk_anchors(FAKE, 1, 10, 3, 0, FAKE, ctypes.byref(m_bad), None) == -1   # K disagrees
    m_ps = Bd.MapArgs(1, 0, 10, 3, 12, 20, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    assert lib.acache_build_maps(FAKE, ctypes.byref(m_ps), None) == -3
    m_null = Bd.MapArgs(1, 0, 10, 3, 16, 20, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None)
    assert lib.acache_build_maps(FAKE, ctypes.byref(m_null), None) == -1
    assert lib.acache_build_maps(None, ctypes.byref(m), None) == -1
    m_empty = Bd.MapArgs(0, 0, 10, 3, 16, 0, None, None, None, None, None, None, None, None, None)
    assert lib.acache_build_maps(None, ctypes.byref(m_empty), None) == 0


def test_scatter_and_attention_validation():
    lib = Bd._lib()
    p = pool()
    sc = lambda **kw: lib.acache_scatter_private(
        ctypes.byref(kw.pop("pool", p)), kw.get("k", FAKE), kw.get("v", FAKE), kw.get("dst", FAKE),
        kw.get("n", 4), kw.get("lb", 0), kw.get("nl", 2), None)
    assert sc(n=0) == 0                     # zero rows: no-op, nothing launched
    assert sc(nl=0) == 0
    assert sc(n=-1) == -1
    assert sc(k=None) == -1
    assert sc(dst=None) == -1
    assert sc(k=FAKE_MIS) == -9
    assert sc(lb=1) == -1
    assert sc(pool=pool(dtype=3)) == -2
    at = lambda **kw: lib.acache_mapped_attention(
        ctypes.byref(p), kw.get("q", FAKE), FAKE, kw.get("nq", 8), kw.get("mq", 8), FAKE, FAKE, 100,
        kw.get("B", 1), kw.get("hq", 2), 0, 2, kw.get("scale", 0.1), kw.get("out", FAKE), None, None, 0, None)
    assert at(B=0) == 0
    assert at(hq=5) == -3
    assert at(mq=9) == -1
    assert at(scale=-1.0) == -1
    assert at(out=None) == -1
    assert at(q=FAKE_MIS) == -9
    assert lib.acache_block_slots(FAKE, FAKE, FAKE, 2, -1, FAKE, None) == -1
    assert lib.acache_block_slots(FAKE, FAKE, FAKE, 0, 32, FAKE, None) == 0
    assert lib.acache_block_slots(None, FAKE, FAKE, 2, 32, FAKE, None) == -1


def test_shared_attention_validation_and_workspace():
    lib = Bd._lib()
    p = pool()
    ws = lambda pl, mq, nl=2, L=64, mkv=100: _ws_query(lib, pl, 3, 96, mq, 4, nl, mkv, L)
    need = ws(p, 32)
    # private lists, counts, exclusion bits
    assert need >= 3 * 100 * 4 + 3 * 4 + 3 * 2 * 4
    assert ws(p, 32, mkv=200) > need and ws(p, 32, L=64000) > need
    assert ws(p, 33) == 0                        # more than 32 rows per request: single-pass path
    assert ws(pool(dtype=0, head_dim=64), 32) == 0
    assert _ws_query(lib, p, 1, 32, 32, 4, 2, 100, 64) == 0   # one request: single-pass path
    at = lambda **kw: lib.acache_mapped_attention_shared(
        ctypes.byref(kw.pop("pool", p)), kw.get("q", FAKE), FAKE, kw.get("nq", 8), kw.get("mq", 8), FAKE, FAKE,
        kw.get("mkv", 100), kw.get("ss", FAKE), kw.get("al", 0), kw.get("L", 64), kw.get("B", 2), kw.get("hq", 4),
        0, 2, kw.get("scale", 0.1), kw.get("out", FAKE), None, kw.get("ws", FAKE * 16), kw.get("wsb", 1 << 24),
        None)
    assert at(B=0) == 0
    assert at(hq=5) == -3
    assert at(mq=9) == -1
    assert at(scale=-1.0) == -1
    assert at(out=None) == -1
    assert at(q=FAKE_MIS) == -9
    assert at(L=-1) == -1 and at(al=-1) == -1
    assert at(ss=None) == -1
    assert at(wsb=16) == -7 and at(ws=None) == -7
    assert at(ws=FAKE + 4) == -9
    assert at(B=70000) == -3
    assert at(B=40000, mkv=60000) == -3          # private lists indexed with 32 bits


def test_store_attend_validation_and_workspace():
    lib = Bd._lib()
    p = pool()

    def ws(pl, B=3, mq=100, mkv=500):
        out = ctypes.c_size_t()
        assert lib.acache_store_attend_workspace_bytes(ctypes.byref(pl), B, mq, mkv, ctypes.byref(out)) == 0
        return out.value
    need = ws(p)
    assert need >= 3 * 500 * 4 + 3 * 4          # other read lists and their counts
    assert ws(p, mkv=1000) > need
    assert ws(p, mq=0) == 0                       # no query rows: the scatter alone
    assert ws(pool(dtype=0, head_dim=64)) == 0    # other pools: the two calls of the definition
    assert ws(p, mkv=(1 << 18) + 1) == 0          # longer contexts: the two calls
    assert ws(p, mq=3072) > 0 and ws(p, mq=3073) == 0   # larger recompute sets: the two calls
    sa = lambda **kw: lib.acache_store_attend(
        ctypes.byref(kw.pop("pool", p)), kw.get("ks", FAKE), kw.get("vs", FAKE), FAKE, FAKE, kw.get("so", FAKE),
        kw.get("ns", 10), kw.get("q", FAKE), FAKE, kw.get("nq", 8), kw.get("mq", 8), FAKE, FAKE, kw.get("mkv", 100),
        kw.get("B", 1), kw.get("hq", 2), 0, 2, kw.get("scale", 0.1), kw.get("out", FAKE), None,
        kw.get("ws", FAKE * 16), kw.get("wsb", 1 << 24), None)
    assert sa(B=0, ns=0) == 0
    assert sa(hq=5) == -3
    assert sa(mq=9) == -1 and sa(ns=-1) == -1
    assert sa(scale=-1.0) == -1
    assert sa(B=70000) == -3
    assert sa(ks=None) == -1 and sa(so=None) == -1
    assert sa(ks=FAKE_MIS) == -9
    assert sa(out=None) == -1
    assert sa(q=FAKE_MIS) == -9
    assert sa(wsb=16) == -7 and sa(ws=None) == -7
    assert sa(ws=FAKE + 4) == -9
    # grouped query heads or more rows per request take the two calls, which
    # need no workspace: the first launch fails instead (EDEVICE, no GPU here)
    assert sa(hq=4, ws=None, wsb=0) == -8
    assert sa(nq=3073, mq=3073, ws=None, wsb=0) == -8


def test_size_limits_rejected_before_any_launch():
    """A pool whose layers exceed the 32-bit byte offsets of the MFMA kernels
    is rejected with ESHAPE by every call that would launch them, before the
    call enqueues anything (its plan or scatter kernels included): on this
    host without a GPU any launch would fail with EDEVICE instead."""
    lib = Bd._lib()
    big = pool(n_pages=1 << 20, n_kv_heads=8)          # 2^20 pages x 8 heads x 4 KiB = 32 GiB per layer
    assert lib.acache_mapped_attention(ctypes.byref(big), FAKE, FAKE, 8, 8, FAKE, FAKE, 100, 1, 8, 0, 2, 0.1, FAKE,
                                       None, None, 0, None) == -3
    ws = ctypes.c_size_t()
    assert lib.acache_mapped_attention_shared_workspace_bytes(ctypes.byref(big), 1, 8, 8, 8, 2, 100, 64,
                                                              ctypes.byref(ws)) == 0
    assert lib.acache_mapped_attention_shared(ctypes.byref(big), FAKE, FAKE, 8, 8, FAKE, FAKE, 100, FAKE, 0, 64, 1, 8,
                                              0, 2, 0.1, FAKE, None, FAKE * 16, max(ws.value, 16), None) == -3
    assert lib.acache_store_attend(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, 10, FAKE, FAKE, 8, 8, FAKE, FAKE,
                                   100, 1, 8, 0, 2, 0.1, FAKE, None, FAKE * 16, 1 << 24, None) == -3
    assert lib.acache_probe_attention(ctypes.byref(big), FAKE, 10, FAKE, 32, 8, 0, 2, 0.1, None, FAKE, None) == -3
    # one page of one layer at 16 MiB (256 KV heads x 256 slots x 256 B): the 24-bit row-offset products overflow
    wide = pool(n_pages=4, page_size=256, n_kv_heads=256)
    assert lib.acache_mapped_attention(ctypes.byref(wide), FAKE, FAKE, 8, 8, FAKE, FAKE, 100, 1, 256, 0, 2, 0.1, FAKE,
                                       None, None, 0, None) == -3
    assert lib.acache_mapped_attention_shared_workspace_bytes(ctypes.byref(wide), 2, 16, 8, 256, 2, 100, 64,
                                                              ctypes.byref(ws)) == 0
    assert lib.acache_mapped_attention_shared(ctypes.byref(wide), FAKE, FAKE, 16, 8, FAKE, FAKE, 100, FAKE, 0, 64, 2,
                                              256, 0, 2, 0.1, FAKE, None, FAKE * 16, max(ws.value, 16), None) == -3
    assert lib.acache_store_attend(ctypes.byref(wide), FAKE, FAKE, FAKE, FAKE, FAKE, 10, FAKE, FAKE, 8, 8, FAKE, FAKE,
                                   100, 1, 256, 0, 2, 0.1, FAKE, None, FAKE * 16, 1 << 24, None) == -3
    assert lib.acache_probe_attention(ctypes.byref(wide), FAKE, 10, FAKE, 32, 256, 0, 2, 0.1, None, FAKE, None) == -3


def _ws_query(lib, pl, B, n_q, mq, hq, nl, mkv, L):
    out = ctypes.c_size_t()
    assert lib.acache_mapped_attention_shared_workspace_bytes(ctypes.byref(pl), B, n_q, mq, hq, nl, mkv, L,
                                                              ctypes.byref(out)) == 0
    return out.value


def test_validate_slots_host_checks():
    ps = 4
    owner = np.array([-1, 0, 0, 1, -2, 1], np.int32)    # page owners: shared, req0, req0, req1, free, req1
    ok = np.array([4, 5, 9, 12, 21], np.int32)
    assert A.acache_validate_slots(ok, owner, 6, ps) == (0, -1)
    assert A.acache_validate_slots(np.array([4, 5, 5], np.int32), owner, 6, ps) == (-6, 2)       # EDUP
    assert A.acache_validate_slots(np.array([4, 5, 5], np.int32), owner, 6, ps, distinct=False)[0] == 0
    assert A.acache_validate_slots(np.array([4, 2], np.int32), owner, 6, ps) == (-5, 1)          # shared page
    assert A.acache_validate_slots(np.array([17], np.int32), owner, 6, ps) == (-5, 0)            # free page
    assert A.acache_validate_slots(np.array([4, 24], np.int32), owner, 6, ps) == (-4, 1)         # out of range
    assert A.acache_validate_slots(np.array([-1], np.int32), owner, 6, ps) == (-4, 0)
    # per-row owners: row 1 must be request 1's
    assert A.acache_validate_slots(np.array([4, 12], np.int32), owner, 6, ps,
                                   owner=np.array([0, 1], np.int32)) == (0, -1)
    assert A.acache_validate_slots(np.array([4, 5], np.int32), owner, 6, ps,
                                   owner=np.array([0, 1], np.int32)) == (-5, 1)


def test_kv_footprint_matches_oracle():
    from oracle import acache_oracle as O
    from synth.configs import WORKLOADS
    for w in WORKLOADS.values():
        K = A.acache_anchor_count(w.L, w.rate)
        seq = [w.T] * w.batch
        got = A.acache_kv_footprint(seq, w.L, K, w.page_size, w.n_layers, w.n_kv_heads, w.head_dim, w.dtype)
        sb = w.n_layers * w.n_kv_heads * w.head_dim * 2 * (4 if w.dtype == "f32" else 2)
        ref = O.kv_footprint(seq, w.L, K, w.page_size, sb)
        assert got == {"shared": ref["shared"], "private": ref["private"], "dense": ref["dense"]}, w.name
    ragged = [70, 65, 99]
    got = A.acache_kv_footprint(ragged, 64, 13, 16, 2, 3, 8, "f32")
    assert got == {k: v for k, v in O.kv_footprint(ragged, 64, 13, 16, 2 * 3 * 8 * 2 * 4).items()
                   if k in ("shared", "private", "dense")}
    assert A.acache_kv_footprint([], 64, 13, 16, 2, 3, 8) == {"shared": 0, "private": 0, "dense": 0}
    for bad in (dict(seq_len=[10], L=64), dict(K=70), dict(page_size=0)):
        a = dict(seq_len=[100], L=64, K=13, page_size=16)
        a.update(bad)
        with pytest.raises(A.AcacheError):
            A.acache_kv_footprint(a["seq_len"], a["L"], a["K"], a["page_size"], 2, 3, 8)
    with pytest.raises(A.AcacheError):
        A.acache_kv_footprint([100], 64, 13, 16, 2, 3, 8, 7)


def test_lse_merge_validation():
    lib = Bd._lib()
    mg = lambda **kw: lib.acache_lse_merge(kw.get("dt", 1), kw.get("n", 4), kw.get("d", 128), kw.get("oa", FAKE),
                                           kw.get("la", FAKE), kw.get("ob", FAKE), kw.get("lb", FAKE),
                                           kw.get("o", FAKE), kw.get("l", FAKE), None)
    assert mg(n=0) == 0
    assert mg(dt=3) == -2
    assert mg(d=96) == -3
    assert mg(n=-1) == -1
    assert mg(la=None) == -1 and mg(l=None) == -1
    assert mg(ob=None) == -1
    assert mg(oa=None, ob=None, o=None, n=0) == 0
    assert mg(o=FAKE_MIS) == -9


def test_hkvd_validation():
    lib = Bd._lib()
    p = pool()
    hk = lambda **kw: lib.acache_hkvd_scores(ctypes.byref(kw.pop("pool", p)), kw.get("ss", FAKE), kw.get("L", 32),
                                             kw.get("kf", FAKE), kw.get("vf", FAKE), kw.get("B", 2),
                                             kw.get("lb", 0), kw.get("nl", 2), kw.get("s", FAKE), None)
    assert hk(B=0) == 0 and hk(L=0) == 0 and hk(nl=0) == 0
    assert hk(B=-1) == -1
    assert hk(lb=1) == -1
    assert hk(ss=None) == -1 and hk(s=None) == -1 and hk(kf=None) == -1
    assert hk(vf=FAKE_MIS) == -9
    assert hk(pool=pool(dtype=4)) == -2


def test_only_the_c_abi_is_exported():
    """The library's dynamic symbol table holds the acache_* calls and nothing
    else (internal kernels, launchers and helpers stay local)."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", Bd.LIB_PATH], capture_output=True, text=True, check=True)
    names = [ln.split()[-1] for ln in out.stdout.splitlines() if ln.strip()]
    assert names and all(n.startswith("acache_") for n in names), [n for n in names if not n.startswith("acache_")]
    assert sorted(names) == declared()


def test_check_slots_validation_and_workspace():
    """Checked mode's pre-pass: sizes, modes, tables and workspace are checked
    on the host before anything is launched; the workspace is 256 bytes for
    reads and 256 + 4 per pool slot (rounded to 256) for writes."""
    lib = Bd._lib()
    nb = ctypes.c_size_t()
    assert lib.acache_check_slots_workspace_bytes(8, 16, A.ACACHE_CHECK_READ, ctypes.byref(nb)) == 0
    assert nb.value == 256
    assert lib.acache_check_slots_workspace_bytes(8, 16, A.ACACHE_CHECK_WRITE, ctypes.byref(nb)) == 0
    assert nb.value == 256 + 512
    assert lib.acache_check_slots_workspace_bytes(100, 16, A.ACACHE_CHECK_WRITE, ctypes.byref(nb)) == 0
    assert nb.value == 256 + 6400
    assert lib.acache_check_slots_workspace_bytes(8, 12, 0, ctypes.byref(nb)) == -1     # page size not a power of 2
    assert lib.acache_check_slots_workspace_bytes(8, 16, 2, ctypes.byref(nb)) == -1     # no such mode
    assert lib.acache_check_slots_workspace_bytes(1 << 28, 16, 1, ctypes.byref(nb)) == -3  # more than 2^31 slots
    bad = ctypes.c_int32(7)
    # (slots, n, offsets, B, page_owner, n_pages, page_size, mode, bad, ws, ws_bytes, stream)
    assert lib.acache_check_slots(FAKE, -1, None, 0, None, 8, 16, 0, ctypes.byref(bad), FAKE, 256, None) == -1
    assert lib.acache_check_slots(None, 4, None, 0, None, 8, 16, 0, ctypes.byref(bad), FAKE, 256, None) == -1
    assert lib.acache_check_slots(FAKE, 4, None, 2, None, 8, 16, 0, ctypes.byref(bad), FAKE, 256, None) == -1
    assert lib.acache_check_slots(FAKE, 4, None, 0, None, 8, 16, 1, ctypes.byref(bad), FAKE, 256, None) == -7
    assert lib.acache_check_slots(FAKE, 4, None, 0, None, 8, 16, 0, ctypes.byref(bad), None, 256, None) == -7
    assert lib.acache_check_slots(FAKE, 4, None, 0, None, 8, 16, 0, ctypes.byref(bad), FAKE + 16, 256, None) == -7
    assert bad.value == 7   # untouched on a host-side error
    p = pool()
    # (pool, k_src, v_src, dst, n_rows, row_offsets, B, page_owner, layer_begin, n_layers, bad, ws, ws_bytes, stream)
    assert lib.acache_scatter_private_checked(ctypes.byref(p), FAKE, FAKE, FAKE, 4, FAKE, 1, FAKE, 0, 3,
                                              ctypes.byref(bad), FAKE, 4096, None) == -1   # layer range
    assert lib.acache_scatter_private_checked(ctypes.byref(p), FAKE_MIS, FAKE, FAKE, 4, FAKE, 1, FAKE, 0, 2,
                                              ctypes.byref(bad), FAKE, 4096, None) == -9
    assert lib.acache_scatter_private_checked(ctypes.byref(p), FAKE, FAKE, FAKE, 4, FAKE, 1, FAKE, 0, 2,
                                              ctypes.byref(bad), FAKE, 512, None) == -7    # write mode needs 768
