"""Seeded sweeps of small random shapes against the oracle.

The probe and the maps (Section 3.2 Eq. 4-6, Section 4.1): probe O_aff, LSE
and scores over 1-3 layers, the Top-K on the library's own scores against a
sort of the same scores (bit-exact), and both maps against the oracle's maps
of those anchors (bit-exact).

The three read-slot attention calls (single pass, shared affix,
store-then-attend; Section 4.3, Appendix C.1): head dims 16-128, grouped query heads
(G = 1..5), page sizes 4-32, bf16 and fp32 pools, ragged query blocks (empty
ones included), contexts of 0 or 1 key, affixes that start anywhere, read
tables with a random share of the affix routed to the shared slots.  Each
case is small; together they reach the kernels' packed and unpacked paths,
partial tiles and every fallback."""
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

N_CASES = 36


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    dtype = "f32" if seed % 6 == 5 else "bf16"
    d = int(rng.choice([16, 32, 64, 128])) if dtype == "f32" or seed % 3 == 0 else 128
    hkv = int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 3, 4, 5]))
    ps = int(rng.choice([4, 8, 16, 32]))
    L = int(rng.integers(1, 300))
    pre = int(rng.integers(0, 40))
    gen_len = int(rng.integers(8, 80))
    B = int(rng.integers(1, 10))
    w = Workload(200 + seed, f"sweep{seed}", dtype, 1, G * hkv, hkv, d,
                 (("req", pre), ("affix", L), ("gen", gen_len)) if pre else (("affix", L), ("gen", gen_len)),
                 B, float(rng.uniform(0.0, 0.6)), page_size=ps, page_order="random")
    return w, rng


@pytest.mark.parametrize("seed", range(N_CASES))
def test_read_slot_attention_sweep(seed):
    w, rng = _case(seed)
    K = A.acache_anchor_count(w.L, w.rate)
    lay = gen.make_layout(w, K, seed)
    k, v = gen.make_pool(w, lay, device=DEV, seed=seed)
    nslot = lay.n_pages * w.page_size
    shared = lay.shared_slots.astype(np.int32)
    # contexts: the maps' full length, a short one, an empty one, one key
    T = [int(w.T)] * w.batch
    for b in range(w.batch):
        r = rng.random()
        T[b] = 0 if r < 0.1 else (1 if r < 0.2 else (int(rng.integers(2, w.T + 1)) if r < 0.4 else w.T))
    share = rng.uniform(0.0, 1.0)
    tables = []
    for b, t in enumerate(T):
        rs = rng.integers(0, nslot, t).astype(np.int32)
        j = np.arange(max(0, min(t - w.affix_l, w.L)))
        keep = rng.random(len(j)) < share
        rs[w.affix_l + j[keep]] = shared[j[keep]]
        tables.append(rs)
    read = np.concatenate(tables).astype(np.int32) if tables else np.zeros(0, np.int32)
    kv_off = np.concatenate([[0], np.cumsum(T)]).astype(np.int32)
    q_counts = [0 if rng.random() < 0.15 else int(rng.integers(1, 70 if rng.random() < 0.3 else 33))
                for _ in range(w.batch)]
    q_off = np.concatenate([[0], np.cumsum(q_counts)]).astype(np.int32)
    n_q = int(q_off[-1])
    if n_q == 0:
        q_counts[0] = 5
        q_off = np.concatenate([[0], np.cumsum(q_counts)]).astype(np.int32)
        n_q = 5
    q = gen.make_rows(w, n_q, gen.S_QDEC, device=DEV, heads=w.n_q_heads, seed=seed)
    # store-then-attend sources: for each request, a random set of its
    # positions whose slots are read exactly there (their own read slots)
    src_pos, src_slot, src_off = [], [], [0]
    slots_all, counts_all = np.unique(read, return_counts=True)
    once = set(slots_all[counts_all == 1].tolist())    # slots read at exactly one position of one request
    for b, t in enumerate(T):
        if t and rng.random() < 0.7:
            pos = np.sort(rng.choice(t, size=int(rng.integers(1, min(t, 40) + 1)), replace=False))
            slots = tables[b][pos]
            # the stored rows' contract: each stored slot is read at its own
            # position and nowhere else
            ok = [p for p, s in zip(pos, slots) if int(s) in once]
            src_pos += [int(p) for p in ok]
            src_slot += [int(tables[b][p]) for p in ok]
        src_off.append(len(src_pos))
    n_src = len(src_pos)
    src_k = gen.make_rows(w, max(n_src, 1), gen.S_SRC_K, device=DEV, seed=seed)[:, :n_src].contiguous()
    src_v = gen.make_rows(w, max(n_src, 1), gen.S_SRC_V, device=DEV, seed=seed)[:, :n_src].contiguous()
    torch.cuda.synchronize()
    kh, vh, qh, skh, svh = map(np_of, (k, v, q, src_k, src_v))
    scale = 1 / math.sqrt(w.head_dim)
    mq, mkv = max(q_counts), max(max(T), 1)
    r_read, r_kv, r_q = i32(read), i32(kv_off), i32(q_off)

    def check(out, lse, kp, vp, what):
        ref, rl = O.mapped_attention_layer(qh[0], kp[0], vp[0], q_off, read, kv_off, w.n_kv_heads, w.page_size,
                                           scale)
        o = np_of(out[0]).astype(np.float64) if w.dtype == "f32" else out[0].float().cpu().numpy()
        live = np.ones(n_q, bool)
        for b, t in enumerate(T):
            if t == 0:
                live[q_off[b]:q_off[b + 1]] = False
        if w.dtype == "f32":
            assert np.abs(o[live] - ref[live]).max(initial=0.0) <= 1e-5, what
        else:
            ok, st = bf16_close(o[live], ref[live])
            assert ok, (what, st)
        assert (o[~live] == 0).all(), what
        lg = lse[0].cpu().numpy()
        assert np.isneginf(lg[~live]).all(), what
        np.testing.assert_allclose(lg[live], rl[live], atol=1e-4, err_msg=what)

    out = torch.full_like(q, 7.0)
    lse = torch.empty(q.shape[:3], device=DEV)
    A.acache_mapped_attention(k, v, q, r_q, r_read, r_kv, out, lse=lse, max_q_per_req=mq, max_kv_per_req=mkv)
    torch.cuda.synchronize()
    check(out, lse, kh, vh, "single pass")
    out.fill_(7.0)
    A.acache_mapped_attention_shared(k, v, q, r_q, r_read, r_kv, i32(shared), out, lse=lse, affix_l=w.affix_l,
                                     max_q_per_req=mq, max_kv_per_req=mkv)
    torch.cuda.synchronize()
    check(out, lse, kh, vh, "shared affix")
    out.fill_(7.0)
    A.acache_store_attend(k, v, src_k, src_v, i32(np.array(src_pos, np.int32)), i32(np.array(src_slot, np.int32)),
                          i32(np.array(src_off, np.int32)), q, r_q, r_read, r_kv, out, lse=lse, max_q_per_req=mq,
                          max_kv_per_req=mkv)
    torch.cuda.synchronize()
    kp, vp = kh.copy(), vh.copy()
    O.scatter(kp, vp, skh, svh, np.array(src_slot, np.int32), w.page_size)
    assert np.array_equal(np_of(k), kp) and np.array_equal(np_of(v), vp), "pool after store-then-attend"
    check(out, lse, kp, vp, "store-then-attend")


@pytest.mark.parametrize("seed", range(24))
def test_probe_and_maps_sweep(seed):
    rng = np.random.default_rng(5000 + seed)
    dtype = "f32" if seed % 5 == 4 else "bf16"
    d = int(rng.choice([16, 32, 64, 128])) if dtype == "f32" or seed % 3 == 0 else 128
    hkv = int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 3, 4, 7]))
    ps = int(rng.choice([4, 8, 16, 32]))
    L = int(rng.integers(1, 400))
    pre, mid = int(rng.integers(0, 50)), int(rng.integers(0, 30))
    m = int(rng.integers(1, 90))
    segs = ([("req", pre)] if pre else []) + [("affix", L)] + ([("req", mid)] if mid else []) + [("gen", m)]
    if rng.random() < 0.3:   # affix as a suffix
        segs = ([("req", pre)] if pre else []) + [("gen", m), ("affix", L)]
    w = Workload(300 + seed, f"psweep{seed}", dtype, int(rng.integers(1, 4)), G * hkv, hkv, d, tuple(segs),
                 int(rng.integers(1, 7)), float(rng.choice([0.0, 0.1, 0.3, 0.5, 1.0])), page_size=ps,
                 page_order="random")
    K = A.acache_anchor_count(w.L, w.rate)
    assert K == O.anchor_count(w.L, w.rate)
    lay = gen.make_layout(w, K, seed)
    k, v = gen.make_pool(w, lay, device=DEV, seed=seed)
    q = gen.make_probe_q(w, lay, device=DEV, seed=seed)
    torch.cuda.synchronize()
    kh, vh, qh = map(np_of, (k, v, q))
    scale = 1 / math.sqrt(w.head_dim)
    scores = torch.zeros((w.batch, w.L), device=DEV)
    o_aff = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], device=DEV)
    A.acache_probe_scores(k, v, q, i32(lay.masked_rows), i32(lay.masked_offsets), i32(lay.shared_slots), scores,
                          max_masked=w.m, o_aff=o_aff, lse_aff=lse)
    n_rc = int(lay.rc_offsets[-1])
    anchors = torch.empty((w.batch, K), dtype=torch.int32, device=DEV)
    read_slot = torch.empty(int(lay.kv_offsets[-1]), dtype=torch.int32, device=DEV)
    rc_pos = torch.empty(max(n_rc, 1), dtype=torch.int32, device=DEV)
    rc_slot = torch.empty_like(rc_pos)
    keep = [i32(x) for x in (lay.seq_len, lay.shared_slots, lay.private_pages, lay.private_page_offsets,
                             lay.kv_offsets, lay.rc_offsets)]
    maps = A.map_args(w.batch, w.affix_l, w.L, K, w.page_size, w.T, *keep, read_slot, rc_pos, rc_slot)
    A.acache_topk_anchors(scores, K, w.affix_l, anchors, maps)
    torch.cuda.synchronize()
    s_gpu = scores.cpu().numpy()
    s_ref = np.zeros((w.batch, w.L))
    for n in range(w.n_layers):
        o_ref, l_ref, s_n = O.probe_layer(qh[n], kh[n], vh[n], lay.shared_slots, w.page_size, w.n_kv_heads,
                                          lay.masked_rows, lay.masked_offsets, scale)
        s_ref += s_n
        o = np_of(o_aff[n]).astype(np.float64) if dtype == "f32" else o_aff[n].float().cpu().numpy()
        if dtype == "f32":
            assert np.abs(o - o_ref).max() <= 1e-5
        else:
            ok, st = bf16_close(o, o_ref)
            assert ok, (n, st)
        np.testing.assert_allclose(lse[n].cpu().numpy(), l_ref, atol=1e-4)
    big = s_ref >= 1e-6 * s_ref.max()
    assert (np.abs(s_gpu - s_ref)[big] / s_ref[big]).max(initial=0.0) <= (1e-5 if dtype == "f32" else 1e-3)
    np.testing.assert_allclose(s_gpu.sum(axis=1), w.n_layers * w.n_q_heads * np.diff(lay.masked_offsets),
                               rtol=1e-4)
    # Top-K on the library's own scores: the same set and order as a sort of
    # those scores (ties to the lower offset), bit for bit
    an = anchors.cpu().numpy()
    rd, rp, rs = [], [], []
    for b in range(w.batch):
        want = O.topk_anchors(s_gpu[b].astype(np.float64), K, w.affix_l)
        assert np.array_equal(an[b], want), f"request {b}"
        pp = lay.private_pages[lay.private_page_offsets[b]:lay.private_page_offsets[b + 1]]
        r_, p_, s_ = O.build_maps(an[b], int(lay.seq_len[b]), w.affix_l, w.L, lay.shared_slots, pp, w.page_size)
        rd.append(r_); rp.append(p_); rs.append(s_)
    assert np.array_equal(read_slot.cpu().numpy(), np.concatenate(rd))
    assert np.array_equal(rc_pos.cpu().numpy()[:n_rc], np.concatenate(rp))
    assert np.array_equal(rc_slot.cpu().numpy()[:n_rc], np.concatenate(rs))


@pytest.mark.parametrize("seed", range(16))
def test_many_query_sweep(seed):
    """Units of at least 384 query rows (the many-query kernel with 48 rows
    per wave): the read-slot attention of ragged query sets (some requests
    with few or no rows, up to 1300) over ragged read tables (0, 1, 31-33
    keys, up to 300; any slot of the pool), with one KV head serving 1-7
    query heads, and the probe of up to 900 non-affix rows over an affix of
    1-260 keys.  Against the oracle's definition of each (Section 4.3,
    Appendix C.1; Section 3.2 Eq. 4)."""
    rng = np.random.default_rng(7000 + seed)
    hkv = int(rng.integers(1, 3))
    G = int(rng.choice([1, 1, 2, 3, 4, 7]))
    ps = int(rng.choice([4, 8, 16, 32]))
    L = int(rng.integers(1, 260))
    B = int(rng.integers(1, 5))
    w = Workload(400 + seed, f"mqsweep{seed}", "bf16", int(rng.integers(1, 3)), G * hkv, hkv, 128,
                 (("affix", L), ("gen", 40)), B, 0.3, page_size=ps, page_order="random")
    K = A.acache_anchor_count(w.L, w.rate)
    lay = gen.make_layout(w, K, seed)
    k, v = gen.make_pool(w, lay, device=DEV, seed=seed)
    nslot = lay.n_pages * w.page_size
    scale = 1 / math.sqrt(w.head_dim)
    # ragged query sets: one request holds at least 384 / G rows, so its
    # units are many-query ones; the others hold 0 to 1300 rows
    need = -(-384 // G)
    q_counts = [int(rng.choice([0, int(rng.integers(1, 40)), int(rng.integers(need, 1300))])) for _ in range(B)]
    q_counts[int(rng.integers(0, B))] = int(rng.integers(need, 1300))
    q_off = np.concatenate([[0], np.cumsum(q_counts)]).astype(np.int32)
    n_q = int(q_off[-1])
    T = [int(rng.choice([0, 1, 31, 32, 33, int(rng.integers(2, 300))])) for _ in range(B)]
    read = np.concatenate([rng.integers(0, nslot, t) for t in T] + [np.zeros(0)]).astype(np.int32)
    kv_off = np.concatenate([[0], np.cumsum(T)]).astype(np.int32)
    q = gen.make_rows(w, n_q, gen.S_QDEC, device=DEV, heads=w.n_q_heads, seed=seed)
    torch.cuda.synchronize()
    kh, vh, qh = map(np_of, (k, v, q))
    out = torch.full_like(q, 7.0)
    lse = torch.empty(q.shape[:3], device=DEV)
    A.acache_mapped_attention(k, v, q, i32(q_off), i32(read), i32(kv_off), out, lse=lse,
                              max_q_per_req=max(q_counts), max_kv_per_req=max(max(T), 1))
    torch.cuda.synchronize()
    for n in range(w.n_layers):
        ref, rl = O.mapped_attention_layer(qh[n], kh[n], vh[n], q_off, read, kv_off, w.n_kv_heads, w.page_size,
                                           scale)
        o = out[n].float().cpu().numpy()
        live = np.ones(n_q, bool)
        for b, t in enumerate(T):
            if t == 0:
                live[q_off[b]:q_off[b + 1]] = False
        ok, st = bf16_close(o[live], ref[live])
        assert ok, (n, st)
        assert (o[~live] == 0).all()
        lg = lse[n].cpu().numpy()
        assert np.isneginf(lg[~live]).all()
        np.testing.assert_allclose(lg[live], rl[live], atol=1e-4)
    # the probe of every non-affix row of a larger batch over the affix
    pq = gen.make_rows(w, int(rng.integers(need, 900)), gen.S_QRC, device=DEV, heads=w.n_q_heads, seed=seed)
    torch.cuda.synchronize()
    pqh = np_of(pq)
    o_aff = torch.empty_like(pq)
    lse_aff = torch.empty(pq.shape[:3], device=DEV)
    A.acache_probe_attention(k, v, pq, i32(lay.shared_slots), lse_aff, o_aff=o_aff)
    torch.cuda.synchronize()
    for n in range(w.n_layers):
        o_ref, l_ref, _ = O.probe_layer(pqh[n], kh[n], vh[n], lay.shared_slots, w.page_size, w.n_kv_heads,
                                        np.zeros(0, np.int64), np.zeros(2, np.int64), scale)
        ok, st = bf16_close(o_aff[n].float().cpu().numpy(), o_ref)
        assert ok, ("probe", n, st)
        np.testing.assert_allclose(lse_aff[n].cpu().numpy(), l_ref, atol=1e-4)
