"""The allocation-free shared-affix call against the call with a workspace.

acache_mapped_attention_shared_noalloc runs the same plan and attention
kernels as acache_mapped_attention_shared, with the plan in the library's
fixed per-GPU scratch array.  Two calls in a row (the second on a smaller
batch, so stale plan entries of the first would show) must equal the
workspace call bit for bit, and their outputs must meet the oracle's bar.
"""
import math

import numpy as np
import pytest
import torch

import attention_anchor_probe_amd as A
from oracle import acache_oracle as O
from synth.configs import Workload
from synth import gen
from tests.gpu_common import DEV, bf16_close, i32
from tests.helpers import np_of

pytestmark = pytest.mark.gpu


def _case(cid, segments, batch, n_q_heads=4, n_kv_heads=4):
    w = Workload(cid, "na", "bf16", 2, n_q_heads, n_kv_heads, 128, segments, batch, 0.2, page_order="random")
    K = O.anchor_count(w.L, w.rate)
    lay = gen.make_layout(w, K, cid)
    k, v = gen.make_pool(w, lay, device=DEV, seed=cid)
    anchors = [O.topk_anchors(np.random.default_rng(cid + b).standard_normal(w.L), K, w.affix_l)
               for b in range(w.batch)]
    read = []
    for b in range(w.batch):
        pp = lay.private_pages[lay.private_page_offsets[b]:lay.private_page_offsets[b + 1]]
        read.append(O.build_maps(anchors[b], int(lay.seq_len[b]), w.affix_l, w.L, lay.shared_slots, pp,
                                 w.page_size)[0])
    n_dec = 32
    qd = gen.make_rows(w, w.batch * n_dec, gen.S_QDEC, device=DEV, seed=cid, heads=w.n_q_heads)
    q_off = np.arange(w.batch + 1) * n_dec
    return w, lay, k, v, np.concatenate(read), qd, q_off


def _run_both(w, lay, k, v, read, qd, q_off):
    args = (k, v, qd, i32(q_off), i32(read), i32(lay.kv_offsets), i32(lay.shared_slots))
    kw = dict(affix_l=w.affix_l, max_q_per_req=32, max_kv_per_req=w.T)
    o_ws, l_ws = torch.empty_like(qd), torch.empty(qd.shape[:3], device=DEV)
    o_na, l_na = torch.full_like(qd, 7.0), torch.full(qd.shape[:3], 7.0, device=DEV)
    A.acache_mapped_attention_shared(*args, o_ws, lse=l_ws, **kw)
    A.acache_mapped_attention_shared_noalloc(*args, o_na, lse=l_na, **kw)
    torch.cuda.synchronize()
    return o_ws, l_ws, o_na, l_na


@pytest.mark.parametrize("gqa", [False, True])
def test_noalloc_matches_the_workspace_call_twice(gqa):
    hq, hkv = (16, 2) if gqa else (4, 4)
    big = _case(131, (("affix", 700), ("req", 40), ("gen", 96)), 6, hq, hkv)
    small = _case(132, (("affix", 190), ("req", 9), ("gen", 40)), 2, hq, hkv)
    for w, lay, k, v, read, qd, q_off in (big, small):
        o_ws, l_ws, o_na, l_na = _run_both(w, lay, k, v, read, qd, q_off)
        assert torch.equal(o_na, o_ws), "O differs from the workspace call"
        assert torch.equal(l_na, l_ws), "LSE differs from the workspace call"
        hk, hv, hq_ = np_of(k), np_of(v), np_of(qd)
        for n in range(w.n_layers):
            ref, rl = O.mapped_attention_layer(hq_[n], hk[n], hv[n], q_off, read, lay.kv_offsets, w.n_kv_heads,
                                               w.page_size, 1 / math.sqrt(w.head_dim))
            ok, st = bf16_close(o_na[n].float().cpu().numpy(), ref)
            assert ok, f"layer {n}: {st}"
            np.testing.assert_allclose(l_na[n].cpu().numpy(), rl, atol=1e-4)


def test_noalloc_refuses_a_plan_beyond_its_scratch():
    w, lay, k, v, read, qd, q_off = _case(133, (("affix", 64), ("req", 8), ("gen", 32)), 3)
    out = torch.full_like(qd, 7.0)
    with pytest.raises(A.AcacheError) as ei:
        # a per-request key bound of 2^20 asks for a 12 MiB plan (3 requests x 4 bytes x 2^20)
        A.acache_mapped_attention_shared_noalloc(k, v, qd, i32(q_off), i32(read), i32(lay.kv_offsets),
                                                 i32(lay.shared_slots), out, affix_l=w.affix_l, max_q_per_req=32,
                                                 max_kv_per_req=1 << 20)
    torch.cuda.synchronize()
    assert ei.value.status == -7
    assert bool((out == 7.0).all()), "nothing may run on a refused call"
