"""Checked mode on the GPU: the device pre-pass over slot tables.

Section 4.1 of "Affix Cache for Diffusion Large Language Models": requests
read the shared region and their own private slots and write only their own
private slots; Appendix C.1: the store writes through the write-side map
before the read-slot attention reads through the read-slot map.  The checked
scatter must refuse out-of-range, shared-region, foreign and duplicate
destinations with the pool left byte-identical, and scatter exactly as the
oracle does when the table is sound.  Every bad slot here is only compared by
the pre-pass, never used as an address.
"""
import numpy as np
import pytest
import torch

import attention_anchor_probe_amd as A
from oracle import acache_oracle as O
from synth.configs import Workload
from synth import gen
from tests.gpu_common import DEV, i32
from tests.helpers import np_of

pytestmark = pytest.mark.gpu

ERANGE, EREGION, EDUP = -4, -5, -6


def _case():
    w = Workload(120, "chk", "bf16", 2, 4, 2, 64, (("req", 5), ("affix", 70), ("gen", 23)), 3, 0.2,
                 page_order="fragmented", free_frac=0.25)
    K = O.anchor_count(w.L, w.rate)
    lay = gen.make_layout(w, K, 5)
    k, v = gen.make_pool(w, lay, device=DEV, seed=5)
    anchors = [O.topk_anchors(np.random.default_rng(b).standard_normal(w.L), K, w.affix_l) for b in range(w.batch)]
    read, rcp, rcs = [], [], []
    for b in range(w.batch):
        pp = lay.private_pages[lay.private_page_offsets[b]:lay.private_page_offsets[b + 1]]
        r_, p_, s_ = O.build_maps(anchors[b], int(lay.seq_len[b]), w.affix_l, w.L, lay.shared_slots, pp, w.page_size)
        read.append(r_); rcp.append(p_); rcs.append(s_)
    n_rc = int(lay.rc_offsets[-1])
    src_k = gen.make_rows(w, n_rc, gen.S_SRC_K, device=DEV, seed=5)
    src_v = gen.make_rows(w, n_rc, gen.S_SRC_V, device=DEV, seed=5)
    return w, lay, k, v, np.concatenate(read), np.concatenate(rcs), src_k, src_v


def _expect_refused(w, lay, k, v, dst, src_k, src_v, status, index):
    k0, v0 = np_of(k), np_of(v)
    with pytest.raises(A.AcacheError) as ei:
        A.acache_scatter_private_checked(k, v, src_k, src_v, i32(dst), i32(lay.rc_offsets), i32(lay.page_owner))
    torch.cuda.synchronize()
    assert ei.value.status == status and ei.value.bad_index == index, (ei.value.status, ei.value.bad_index)
    assert np.array_equal(np_of(k), k0) and np.array_equal(np_of(v), v0), "the pool changed on a refused call"


def test_checked_scatter_refuses_bad_destinations_and_leaves_the_pool():
    w, lay, k, v, read, rcs, src_k, src_v = _case()
    n_slots = lay.n_pages * w.page_size
    shared = int(lay.shared_slots[3])
    # a destination past the pool, and a negative one
    for i, bad in ((6, n_slots + 3), (11, -1), (0, n_slots)):
        d = rcs.copy(); d[i] = bad
        _expect_refused(w, lay, k, v, d, src_k, src_v, ERANGE, i)
    # the shared region, and a page of another request
    d = rcs.copy(); d[9] = shared
    _expect_refused(w, lay, k, v, d, src_k, src_v, EREGION, 9)
    r1 = int(lay.rc_offsets[1])
    d = rcs.copy(); d[r1 + 2] = rcs[4]     # request 1 writes request 0's slot (also a duplicate: EREGION first)
    _expect_refused(w, lay, k, v, d, src_k, src_v, EREGION, r1 + 2)
    free_pages = np.flatnonzero(lay.page_owner == -2)
    assert len(free_pages) > 0
    d = rcs.copy(); d[5] = int(free_pages[0]) * w.page_size + 1
    _expect_refused(w, lay, k, v, d, src_k, src_v, EREGION, 5)
    # a slot named twice inside one request: the later entry is reported
    d = rcs.copy(); d[8] = rcs[2]
    _expect_refused(w, lay, k, v, d, src_k, src_v, EDUP, 8)
    # several classes at once: the first class in the order ERANGE, EREGION, EDUP, smallest entry
    d = rcs.copy(); d[3] = shared; d[7] = n_slots + 100; d[12] = n_slots + 1; d[10] = rcs[1]
    _expect_refused(w, lay, k, v, d, src_k, src_v, ERANGE, 7)
    # a sound table: the checked call scatters exactly as the oracle does
    hk, hv, hsk, hsv = np_of(k), np_of(v), np_of(src_k), np_of(src_v)
    A.acache_scatter_private_checked(k, v, src_k, src_v, i32(rcs), i32(lay.rc_offsets), i32(lay.page_owner))
    torch.cuda.synchronize()
    O.scatter(hk, hv, hsk, hsv, rcs, w.page_size)
    assert np.array_equal(np_of(k), hk) and np.array_equal(np_of(v), hv)


def test_check_slots_read_tables():
    """Read mode: every slot in range and in a shared page or a page of its
    own request; a table of the shared region alone (no segments) must stay
    in shared pages; a broken offsets table is an ERANGE at entry -1."""
    w, lay, k, v, read, rcs, src_k, src_v = _case()
    npg, ps = lay.n_pages, w.page_size
    po, ko = i32(lay.page_owner), i32(lay.kv_offsets)
    R = A.ACACHE_CHECK_READ
    assert A.acache_check_slots(i32(read), npg, ps, R, offsets=ko, page_owner=po) == (0, -2)
    assert A.acache_check_slots(i32(lay.shared_slots), npg, ps, R, page_owner=po) == (0, -2)
    # without page owners only the ranges are checked
    assert A.acache_check_slots(i32(read), npg, ps, R, offsets=ko) == (0, -2)
    b1 = int(lay.kv_offsets[1])
    bad = read.copy(); bad[b1 + 4] = rcs[0]                    # request 1 reads request 0's private slot
    assert A.acache_check_slots(i32(bad), npg, ps, R, offsets=ko, page_owner=po) == (EREGION, b1 + 4)
    bad = read.copy(); bad[17] = npg * ps
    assert A.acache_check_slots(i32(bad), npg, ps, R, offsets=ko, page_owner=po) == (ERANGE, 17)
    assert A.acache_check_slots(i32(bad), npg, ps, R, offsets=ko) == (ERANGE, 17)
    ss = lay.shared_slots.copy(); ss[20] = rcs[3]
    assert A.acache_check_slots(i32(ss), npg, ps, R, page_owner=po) == (EREGION, 20)
    bad_off = lay.kv_offsets.copy(); bad_off[1], bad_off[2] = bad_off[2], bad_off[1]
    assert A.acache_check_slots(i32(read), npg, ps, R, offsets=i32(bad_off), page_owner=po)[0] == ERANGE
    bad_off = lay.kv_offsets.copy(); bad_off[-1] -= 1
    assert A.acache_check_slots(i32(read), npg, ps, R, offsets=i32(bad_off), page_owner=po) == (ERANGE, -1)
    # reads may repeat a slot (the write mode forbids it)
    rep = read.copy(); rep[2] = rep[1]
    assert A.acache_check_slots(i32(rep), npg, ps, R, offsets=ko, page_owner=po)[0] == 0
    assert A.acache_check_slots(i32(rep), npg, ps, A.ACACHE_CHECK_WRITE, offsets=ko)[0] == EDUP


def test_check_slots_on_a_second_call_with_a_smaller_table():
    """The pre-pass clears its own workspace: a failing call followed by a
    sound one on the same workspace reports OK."""
    w, lay, k, v, read, rcs, src_k, src_v = _case()
    npg, ps = lay.n_pages, w.page_size
    W = A.ACACHE_CHECK_WRITE
    ws = torch.empty(256 + -(-npg * ps * 4 // 256) * 256, dtype=torch.uint8, device=DEV)
    d = rcs.copy(); d[4] = d[1]
    assert A.acache_check_slots(i32(d), npg, ps, W, offsets=i32(lay.rc_offsets), workspace=ws) == (EDUP, 4)
    r1 = int(lay.rc_offsets[1])
    assert A.acache_check_slots(i32(rcs[:r1]), npg, ps, W, offsets=i32(lay.rc_offsets[:2]), workspace=ws,
                                page_owner=i32(lay.page_owner)) == (0, -2)
