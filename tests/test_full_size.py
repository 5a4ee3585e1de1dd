"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (every call covers all layers of the workload), checked on
sampled outputs the fp64 oracle computes one by one, plus invariants that hold
at any size.

Per workload (L=1024 probe; Dream-shaped infix L=2048 x 16 requests; L=4096 x
16 requests; L=16384 suffix x 32 requests with 8 decode steps):

Part A -- probe (Eq. 4-5) and Top-K (Eq. 6) on the seeded inputs
  * sum_j scores[b][j] = N * Hq * m for every request (every masked row's
    affix mass is one);
  * per-layer scores of sampled layers (the same kernels launched for that
    layer alone) against the oracle for sampled requests;
  * O_aff and LSE_aff of sampled rows of sampled layers against the oracle;
  * the anchor set of one sampled request against the oracle's Top-K of its
    own full-layer scores (exact beyond the 1e-3 tie band), on every workload;
    at L=16384 that is ~10^12 fp64 operations, about a minute and a half of
    host time, over a host copy of the shared pages (4.3 GB of affix keys).
Part B -- maps, scatter, decode blocks and read-slot attention
  * anchors from a seeded Top-K (the same seeded scores on both sides; the
    library's Top-K must equal the oracle's bit for bit);
  * read-slot map, recompute map and block slots: bit-exact for all requests;
  * the pool after the admission scatter and each block store: bit-exact on
    sampled layers (whole layer, including every untouched byte);
  * the recompute phase on sampled layers: the recomputed rows' attention
    over their full read lists, then the one-call store-then-attend of a
    fresh set of rows (the whole pool layer bit-exact, sampled rows' O and LSE);
  * read-slot attention of sampled (layer, request) pairs at every step.
"""
import math

import numpy as np
import pytest
import torch

import attention_anchor_probe_amd as A
from oracle import acache_oracle as O
from synth.configs import WORKLOADS
from synth import gen
from tests.gpu_common import DEV, anchors_match, bf16_close, i32
from tests.helpers import np_of

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[full-size] {msg}", flush=True)


def _sampled(n, k, seed):
    return sorted(np.random.default_rng(seed).choice(n, size=min(k, n), replace=False).tolist())


def _shared_page_view(w, lay, pool):
    """Host copy of the shared pages of every layer (an input subset) and
    the affix slots renumbered onto it."""
    pages = torch.as_tensor(lay.shared_pages.astype(np.int64), device=DEV)
    sub = np_of(pool.index_select(1, pages))
    remap = {int(p): i for i, p in enumerate(lay.shared_pages)}
    slots = np.array([remap[int(s) // w.page_size] * w.page_size + int(s) % w.page_size for s in lay.shared_slots])
    return sub, slots


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_full_size(cid):
    w = WORKLOADS[cid]
    scale = 1.0 / math.sqrt(w.head_dim)
    K = A.acache_anchor_count(w.L, w.rate)
    assert K == O.anchor_count(w.L, w.rate)
    say(f"workload {cid} {w.name}: N={w.n_layers} Hq={w.n_q_heads} Hkv={w.n_kv_heads} L={w.L} T={w.T} "
        f"B={w.batch} K={K}: generating inputs")
    lay = gen.make_layout(w, K, seed=0)
    k, v = gen.make_pool(w, lay, device=DEV)
    q = gen.make_probe_q(w, lay, device=DEV)
    layers = _sampled(w.n_layers, 2, 100 + cid)
    reqs = _sampled(w.batch, 4, 200 + cid)
    # host snapshots of inputs, taken before the library runs
    hk = {n: np_of(k[n]) for n in layers}
    hv = {n: np_of(v[n]) for n in layers}
    hq = {n: np_of(q[n]) for n in layers}
    full_req = reqs[0]
    shared_k, shared_slots_sub = _shared_page_view(w, lay, k)
    mrow = lay.masked_rows[lay.masked_offsets[full_req]:lay.masked_offsets[full_req + 1]]
    hq_full = np_of(q[:, torch.as_tensor(mrow.astype(np.int64), device=DEV)])
    torch.cuda.synchronize()

    # ------------------------------------------------------------ Part A
    say("probe attention + column mass (all layers)")
    scores = torch.zeros((w.batch, w.L), device=DEV)
    o_aff = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], device=DEV)
    mrows, moffs, sslots = i32(lay.masked_rows), i32(lay.masked_offsets), i32(lay.shared_slots)
    A.acache_probe_attention(k, v, q, sslots, lse, o_aff=o_aff)
    A.acache_probe_column_mass(k, v, q, mrows, moffs, sslots, lse, scores, max_masked=w.m)
    per_layer = {}
    for n in layers:
        s_n = torch.zeros((w.batch, w.L), device=DEV)
        A.acache_probe_column_mass(k, v, q[n:n + 1], mrows, moffs, sslots, lse[n:n + 1], s_n, max_masked=w.m,
                                   layer_begin=n)
        per_layer[n] = s_n
    torch.cuda.synchronize()
    s_gpu = scores.cpu().numpy().astype(np.float64)
    tot = w.n_layers * w.n_q_heads * w.m
    np.testing.assert_allclose(s_gpu.sum(axis=1), tot, rtol=1e-4)
    say("score totals ok; per-layer scores and O_aff/LSE vs oracle")
    for n in layers:
        rows, offs = [], [0]
        for b in reqs:
            rows.append(lay.masked_rows[lay.masked_offsets[b]:lay.masked_offsets[b + 1]])
            offs.append(offs[-1] + len(rows[-1]))
        rows = np.concatenate(rows)
        _, _, s_ref = O.probe_layer(hq[n][rows], hk[n], hv[n], lay.shared_slots, w.page_size, w.n_kv_heads,
                                    np.arange(len(rows)), np.array(offs), scale, want_out=False)
        s_l = per_layer[n].cpu().numpy().astype(np.float64)[reqs]
        big = s_ref >= 1e-6 * s_ref.max()
        rel = (np.abs(s_l - s_ref)[big] / s_ref[big]).max()
        assert rel <= 1e-3, f"layer {n} scores rel err {rel}"
        sample_rows = np.array(_sampled(q.shape[1], 96, 300 + n))
        o_ref, l_ref, _ = O.probe_layer(hq[n][sample_rows], hk[n], hv[n], lay.shared_slots, w.page_size,
                                        w.n_kv_heads, np.zeros(0, np.int64), np.array([0, 0]), scale)
        ok, st = bf16_close(o_aff[n][torch.as_tensor(sample_rows, device=DEV)].float().cpu().numpy(), o_ref)
        assert ok, f"O_aff layer {n}: {st}"
        np.testing.assert_allclose(lse[n][torch.as_tensor(sample_rows, device=DEV)].cpu().numpy(), l_ref, atol=1e-4)
    anchors = torch.empty((w.batch, K), dtype=torch.int32, device=DEV)
    A.acache_topk_anchors(scores, K, w.affix_l, anchors)
    torch.cuda.synchronize()
    an = anchors.cpu().numpy()
    for b in range(w.batch):
        assert len(set(an[b].tolist())) == K and (np.diff(an[b]) > 0).all()
        assert an[b][0] >= w.affix_l and an[b][-1] < w.affix_l + w.L
    say(f"anchor set of request {full_req} vs the oracle's full-layer scores")
    s_full = O.probe_scores(hq_full, shared_k, shared_k, shared_slots_sub, w.page_size, w.n_kv_heads,
                            np.arange(w.m), np.array([0, w.m]), scale)[0]
    ok, exact = anchors_match(s_full, an[full_req], K, w.affix_l)
    assert ok, "anchor set differs from the oracle beyond the tie band"
    big = s_full >= 1e-6 * s_full.max()
    rel = (np.abs(s_gpu[full_req] - s_full)[big] / s_full[big]).max()
    assert rel <= 1e-3, f"request {full_req} scores rel err {rel}"
    say(f"anchor set of request {full_req}: {'exact' if exact else 'within the tie band'}, scores rel err {rel:.2e}")
    del o_aff, lse, per_layer, shared_k, hq_full

    # ------------------------------------------------------------ Part B
    say("seeded Top-K + maps")
    s_seed = gen.seeded_scores(w, device=DEV)
    hs_seed = s_seed.cpu().numpy().astype(np.float64)
    an_ref = [O.topk_anchors(hs_seed[b], K, w.affix_l) for b in range(w.batch)]
    n_rc = int(lay.rc_offsets[-1])
    read = torch.empty(int(lay.kv_offsets[-1]), dtype=torch.int32, device=DEV)
    rcp = torch.empty(n_rc, dtype=torch.int32, device=DEV)
    rcs = torch.empty_like(rcp)
    keep = [i32(x) for x in (lay.seq_len, lay.shared_slots, lay.private_pages, lay.private_page_offsets,
                             lay.kv_offsets, lay.rc_offsets)]
    maps = A.map_args(w.batch, w.affix_l, w.L, K, w.page_size, w.T, *keep, read, rcp, rcs)
    A.acache_topk_anchors(s_seed, K, w.affix_l, anchors, maps)
    torch.cuda.synchronize()
    assert np.array_equal(anchors.cpu().numpy(), np.array(an_ref))
    rd, rp, rs = [], [], []
    for b in range(w.batch):
        pp = lay.private_pages[lay.private_page_offsets[b]:lay.private_page_offsets[b + 1]]
        r_, p_, s_ = O.build_maps(an_ref[b], w.T, w.affix_l, w.L, lay.shared_slots, pp, w.page_size)
        rd.append(r_); rp.append(p_); rs.append(s_)
    r_read, r_rcpos, r_rcslot = map(np.concatenate, (rd, rp, rs))
    assert np.array_equal(read.cpu().numpy(), r_read)
    assert np.array_equal(rcp.cpu().numpy(), r_rcpos)
    assert np.array_equal(rcs.cpu().numpy(), r_rcslot)
    del q, scores
    say("admission scatter (all layers)")
    src_k = gen.make_rows(w, n_rc, gen.S_SRC_K, device=DEV)
    src_v = gen.make_rows(w, n_rc, gen.S_SRC_V, device=DEV)
    hsk = {n: np_of(src_k[n]) for n in layers}
    hsv = {n: np_of(src_v[n]) for n in layers}
    A.acache_scatter_private(k, v, src_k, src_v, rcs)
    torch.cuda.synchronize()
    del src_k, src_v
    for n in layers:
        O.scatter(hk[n][None], hv[n][None], hsk[n][None], hsv[n][None], r_rcslot, w.page_size)
        assert np.array_equal(np_of(k[n]), hk[n]) and np.array_equal(np_of(v[n]), hv[n]), f"pool layer {n}"
    del hsk, hsv
    say("recompute-phase read-slot attention: the recomputed rows of every request over their full read lists")
    # queries only for the recomputed positions, keys and values through the read-slot map (Section 4.3)
    max_r = int(np.diff(lay.rc_offsets).max())
    for n in layers:
        qr = gen.make_rows(w, n_rc, gen.S_QRC, device=DEV, heads=w.n_q_heads, layers=[n])
        orc = torch.empty_like(qr)
        lrc = torch.empty(qr.shape[:3], device=DEV)
        A.acache_mapped_attention(k, v, qr, keep[5], read, keep[4], orc, lse=lrc, layer_begin=n,
                                  max_q_per_req=max_r, max_kv_per_req=w.T)
        torch.cuda.synchronize()
        hqr = np_of(qr[0])
        for b in reqs:
            r0, r1 = int(lay.rc_offsets[b]), int(lay.rc_offsets[b + 1])
            rows = r0 + np.array(_sampled(r1 - r0, 48, 400 + b + n))
            o_ref, l_ref = O.mapped_attention_layer(hqr[rows], hk[n], hv[n], [0, len(rows)],
                                                    r_read[lay.kv_offsets[b]:lay.kv_offsets[b + 1]], [0, w.T],
                                                    w.n_kv_heads, w.page_size, scale)
            sel = torch.as_tensor(rows, device=DEV)
            ok, st = bf16_close(orc[0][sel].float().cpu().numpy(), o_ref)
            assert ok, f"recompute-phase attention layer {n} request {b}: {st}"
            np.testing.assert_allclose(lrc[0][sel].cpu().numpy(), l_ref, rtol=2e-5, atol=1e-4)
        # the same queries through the one-call store-then-attend, storing a
        # fresh set of recomputed rows: the pool layer equals the oracle's
        # scatter of them and the attention reads them
        say(f"store-then-attend, layer {n}")
        s2k = gen.make_rows(w, n_rc, gen.S_SRC_K, device=DEV, layers=[n], step=1)
        s2v = gen.make_rows(w, n_rc, gen.S_SRC_V, device=DEV, layers=[n], step=1)
        torch.cuda.synchronize()
        h2k, h2v = np_of(s2k), np_of(s2v)
        A.acache_store_attend(k, v, s2k, s2v, rcp, rcs, keep[5], qr, keep[5], read, keep[4], orc, lse=lrc,
                              layer_begin=n, max_q_per_req=max_r, max_kv_per_req=w.T)
        torch.cuda.synchronize()
        O.scatter(hk[n][None], hv[n][None], h2k, h2v, r_rcslot, w.page_size)
        assert np.array_equal(np_of(k[n]), hk[n]) and np.array_equal(np_of(v[n]), hv[n]), f"stored pool layer {n}"
        for b in reqs:
            r0, r1 = int(lay.rc_offsets[b]), int(lay.rc_offsets[b + 1])
            rows = r0 + np.array(_sampled(r1 - r0, 48, 500 + b + n))
            o_ref, l_ref = O.mapped_attention_layer(hqr[rows], hk[n], hv[n], [0, len(rows)],
                                                    r_read[lay.kv_offsets[b]:lay.kv_offsets[b + 1]], [0, w.T],
                                                    w.n_kv_heads, w.page_size, scale)
            sel = torch.as_tensor(rows, device=DEV)
            ok, st = bf16_close(orc[0][sel].float().cpu().numpy(), o_ref)
            assert ok, f"store-then-attend layer {n} request {b}: {st}"
            np.testing.assert_allclose(lrc[0][sel].cpu().numpy(), l_ref, rtol=2e-5, atol=1e-4)
        del qr, orc, lrc, s2k, s2v
    q_off = np.arange(w.batch + 1) * w.block_len
    for step in range(w.steps):
        say(f"decode step {step}: block slots, block store, read-slot attention (all layers)")
        nb = w.batch * w.block_len
        qd = gen.make_rows(w, nb, gen.S_QDEC, device=DEV, heads=w.n_q_heads, step=step)
        bk = gen.make_rows(w, nb, gen.S_BLK_K, device=DEV, step=step)
        bv = gen.make_rows(w, nb, gen.S_BLK_V, device=DEV, step=step)
        hqd = {n: np_of(qd[n]) for n in layers}
        hbk = {n: np_of(bk[n]) for n in layers}
        hbv = {n: np_of(bv[n]) for n in layers}
        bstart = np.full(w.batch, gen.block_positions(w, step)[0], np.int32)
        dst = torch.empty(nb, dtype=torch.int32, device=DEV)
        A.acache_block_slots(read, keep[4], i32(bstart), w.block_len, dst)
        A.acache_scatter_private(k, v, bk, bv, dst)
        out = torch.empty_like(qd)
        A.acache_mapped_attention(k, v, qd, i32(q_off), read, keep[4], out, max_q_per_req=w.block_len,
                                  max_kv_per_req=w.T)
        out_sh = torch.empty_like(qd)
        lse_sh = torch.empty(qd.shape[:3], device=DEV)
        A.acache_mapped_attention_shared(k, v, qd, i32(q_off), read, keep[4], keep[1], out_sh, lse=lse_sh,
                                         affix_l=w.affix_l, max_q_per_req=w.block_len, max_kv_per_req=w.T)
        torch.cuda.synchronize()
        r_dst = O.block_slots(r_read, lay.kv_offsets, bstart, w.block_len)
        assert np.array_equal(dst.cpu().numpy(), r_dst)
        for n in layers:
            O.scatter(hk[n][None], hv[n][None], hbk[n][None], hbv[n][None], r_dst, w.page_size)
            if step == 0 or step == w.steps - 1:
                assert np.array_equal(np_of(k[n]), hk[n]) and np.array_equal(np_of(v[n]), hv[n])
            for b in reqs:
                qsl = slice(q_off[b], q_off[b + 1])
                o_ref, l_ref = O.mapped_attention_layer(hqd[n][qsl], hk[n], hv[n], [0, w.block_len],
                                                        r_read[lay.kv_offsets[b]:lay.kv_offsets[b + 1]],
                                                        [0, w.T], w.n_kv_heads, w.page_size, scale)
                ok, st = bf16_close(out[n][qsl].float().cpu().numpy(), o_ref)
                assert ok, f"read-slot attention layer {n} request {b} step {step}: {st}"
                ok, st = bf16_close(out_sh[n][qsl].float().cpu().numpy(), o_ref)
                assert ok, f"shared-affix read-slot attention layer {n} request {b} step {step}: {st}"
                # the LSE error follows the fp32 error of the dominant logits, which grows with
                # their size (heavy-tailed keys): 1e-4 plus 2e-5 of the value
                np.testing.assert_allclose(lse_sh[n][qsl].cpu().numpy(), l_ref, rtol=2e-5, atol=1e-4)
        del qd, bk, bv, out, out_sh, lse_sh
    say("done")
