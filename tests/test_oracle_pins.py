"""Pins of the fp64 oracle against what the paper and the mathematics fix.

Nothing here compares the oracle with itself: each check is a hand-worked
fixture, a closed form, an invariant, a library routine the method reduces to
in a special case, or an independent brute-force formulation (oracle/brute.py).
Source: "Affix Cache for Diffusion Large Language Models" (ACache).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import acache_oracle as O
from oracle import brute
from synth.configs import WORKLOADS, Workload
from synth import gen
from tests.helpers import np_of, frac

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def tiny_workload(**kw):
    base = dict(cid=90, name="tiny", dtype="f32", n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=8,
                segments=(("req", 3), ("affix", 11), ("req", 2), ("gen", 5)), batch=2, rate=0.3,
                page_size=4, page_order="random")
    base.update(kw)
    return Workload(**base)


def build_case(w, seed=0, K=None, page_order=None, shared_slot_order=None):
    K = O.anchor_count(w.L, w.rate) if K is None else K
    lay = gen.make_layout(w, K, seed, page_order=page_order, shared_slot_order=shared_slot_order)
    k, v = gen.make_pool(w, lay, seed=seed)
    q = gen.make_probe_q(w, lay, seed=seed)
    return K, lay, np_of(k), np_of(v), np_of(q)


def full_maps(w, K, lay, anchors):
    read, rcp, rcs = [], [], []
    for b in range(w.batch):
        pp = lay.private_pages[lay.private_page_offsets[b]:lay.private_page_offsets[b + 1]]
        r, p, s = O.build_maps(anchors[b], int(lay.seq_len[b]), w.affix_l, w.L, lay.shared_slots, pp,
                               w.page_size)
        read.append(r); rcp.append(p); rcs.append(s)
    return np.concatenate(read), np.concatenate(rcp), np.concatenate(rcs)


# ---------------------------------------------------------------------------
# hand-worked fixtures
# ---------------------------------------------------------------------------
def _golden_probe_inputs(g):
    N, H, d, L = g["n_layers"], g["n_heads"], g["head_dim"], g["L"]
    ps = 4
    q = np.zeros((N, g["rows"], H, d))
    q[..., 0] = math.sqrt(d)
    kp = np.zeros((N, 1, H, ps, d))
    vp = np.zeros((N, 1, H, ps, d))
    for n in range(N):
        for h in range(H):
            for j in range(L):
                kp[n, 0, h, j, 0] = math.log(g["weights"][n][h][j])
    return q, kp, vp, np.arange(L), ps


def test_golden_probe_eq4_eq5():
    g = gold("probe_eq4_eq5.json")
    q, kp, vp, slots, ps = _golden_probe_inputs(g)
    d = g["head_dim"]
    mr, mo = np.array(g["masked_rows"]), np.array(g["masked_offsets"])
    s = O.probe_scores(q, kp, vp, slots, ps, g["n_heads"], mr, mo, 1.0 / math.sqrt(d))
    exp = np.array([[frac(x) for x in row] for row in g["expected_scores"]])
    np.testing.assert_allclose(s, exp, rtol=0, atol=1e-12)
    # the single-layer weights of (layer 0, head 0)
    _, lse, _ = O.probe_layer(q[0], kp[0], vp[0], slots, ps, g["n_heads"], mr, mo, 1.0 / math.sqrt(d))
    w0 = np.exp(np.log(np.array(g["weights"][0][0], float)) - lse[1, 0])
    np.testing.assert_allclose(w0, [frac(x) for x in g["expected_weight_layer0_head0"]], atol=1e-12)
    bs, _, _ = brute.probe(q.tolist(), kp, vp, slots, ps, g["n_heads"], mr, mo, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(np.array(bs), exp, atol=1e-12)


@pytest.mark.parametrize("name", ["maps_prefix.json", "maps_infix.json"])
def test_golden_maps(name):
    g = gold(name)
    r, p, s = O.build_maps(g["anchors"], g["T"], g["affix_l"], g["L"], g["shared_slots"], g["private_pages"],
                           g["page_size"])
    assert r.tolist() == g["read_slot"]
    assert p.tolist() == g["recompute_pos"]
    assert s.tolist() == g["recompute_slot"]
    br, bp, bs = brute.maps(g["anchors"], g["T"], g["affix_l"], g["L"], g["shared_slots"], g["private_pages"],
                            g["page_size"])
    assert br == g["read_slot"] and bp == g["recompute_pos"] and bs == g["recompute_slot"]


def test_golden_topk_ties():
    g = gold("topk_ties.json")
    for k, exp in g["cases"].items():
        assert O.topk_anchors(np.array(g["scores"]), int(k), g["affix_l"]).tolist() == exp
        assert brute.topk(g["scores"], int(k), g["affix_l"]) == exp


def test_golden_mapped_attention():
    g = gold("mapped_attention.json")
    ps, npg, d = g["page_size"], g["n_pages"], 2
    kp = np.zeros((npg, 1, ps, d))
    vp = np.zeros((npg, 1, ps, d))
    for s, w in g["key_weights"].items():
        s = int(s)
        kp[s // ps, 0, s % ps, 0] = math.log(w)
        vp[s // ps, 0, s % ps] = g["values"][str(s)]
    q = np.zeros((1, 1, d)); q[0, 0, 0] = math.sqrt(d)
    o, _ = O.mapped_attention_layer(q, kp, vp, [0, 1], np.array(g["read_slot"]), [0, 3], 1, ps,
                                    1.0 / math.sqrt(d))
    np.testing.assert_allclose(o[0, 0], [frac(x) for x in g["expected_out"]], atol=1e-12)
    bo = brute.mapped_attention([q.tolist()], [kp], [vp], [0, 1], g["read_slot"], [0, 3], 1, ps,
                                1.0 / math.sqrt(d))
    np.testing.assert_allclose(bo[0][0][0], [frac(x) for x in g["expected_out"]], atol=1e-12)


def _block_slots_pins_hold():
    """O.block_slots against its two pins: the hand-worked fixture, and the
    closed-form private slots (oracle/brute.py, no read-slot table) of decode
    blocks in seeded layouts with the affix as prefix, infix and suffix."""
    g = gold("block_slots.json")
    for c in g["cases"]:
        got = O.block_slots(np.array(g["read_slot"]), g["kv_offsets"], c["block_start"], g["block_len"])
        if got.tolist() != c["dst_slots"]:
            return False
    rng = np.random.default_rng(11)
    for segs in ((("affix", 13), ("req", 3), ("gen", 8)), (("req", 2), ("affix", 9), ("req", 3), ("gen", 8)),
                 (("req", 4), ("gen", 8), ("affix", 10))):
        w = tiny_workload(segments=segs, batch=3, page_size=4)
        K = O.anchor_count(w.L, w.rate)
        lay = gen.make_layout(w, K, 3)
        anchors = [O.topk_anchors(rng.standard_normal(w.L), K, w.affix_l) for _ in range(w.batch)]
        read, _, _ = full_maps(w, K, lay, anchors)
        pages = [lay.private_pages[lay.private_page_offsets[b]:lay.private_page_offsets[b + 1]]
                 for b in range(w.batch)]
        gen_pos = [p for p in range(w.T) if not (w.affix_l <= p < w.affix_l + w.L)]
        blen = 4
        starts = [p for p in gen_pos if all(q in gen_pos for q in range(p, p + blen))]
        for _ in range(6):
            bs = [int(rng.choice(starts)) for _ in range(w.batch)]
            got = O.block_slots(read, lay.kv_offsets, bs, blen)
            if got.tolist() != brute.block_slots(anchors, w.affix_l, w.L, pages, w.page_size, bs, blen):
                return False
    return True


def test_golden_block_slots():
    g = gold("block_slots.json")
    pre, inf = gold("maps_prefix.json"), gold("maps_infix.json")
    for c in g["cases"]:
        got = O.block_slots(np.array(g["read_slot"]), g["kv_offsets"], c["block_start"], g["block_len"])
        assert got.tolist() == c["dst_slots"]
    # the closed form reaches the same slots from the anchors and private pages alone
    assert pre["page_size"] == 4 and inf["page_size"] == 2
    for c in g["cases"]:
        b0 = brute.block_slots([pre["anchors"]], pre["affix_l"], pre["L"], [pre["private_pages"]], 4,
                               [c["block_start"][0]], g["block_len"])
        b1 = brute.block_slots([inf["anchors"]], inf["affix_l"], inf["L"], [inf["private_pages"]], 2,
                               [c["block_start"][1]], g["block_len"])
        assert b0 + b1 == c["dst_slots"]


def test_block_slots_closed_form():
    """Decode-block destinations read through the joint read-slot table equal
    the closed-form private slots of the block's positions (Section 4.3 block
    decoding, Section 4.1 maps), in all three affix placements."""
    assert _block_slots_pins_hold()


def _lse_merge_empty_pins_hold():
    """An attention over the empty key set is O = 0, LSE = -inf (the empty
    sum).  Merging it with the attention over a key set S is the attention
    over the union, which is S itself: that part comes back unchanged, in
    either order; two empty parts merge to the empty attention."""
    w = tiny_workload()
    K, lay, k, v, q = build_case(w)
    qd = np_of(gen.make_rows(w, 3, gen.S_QDEC, heads=w.n_q_heads))
    scale = 1 / math.sqrt(w.head_dim)
    keys = lay.shared_slots[:7]
    o_s, l_s = O.mapped_attention_layer(qd[0], k[0], v[0], [0, 3], keys, [0, 7], w.n_kv_heads, w.page_size, scale)
    o_e, l_e = O.mapped_attention_layer(qd[0], k[0], v[0], [0, 3], keys[:0], [0, 0], w.n_kv_heads, w.page_size,
                                        scale)
    if not ((o_e == 0).all() and np.isneginf(l_e).all() and np.isfinite(l_s).all()):
        return False
    for a, b in (((o_e, l_e), (o_s, l_s)), ((o_s, l_s), (o_e, l_e))):
        om, lm = O.lse_merge(a[0], a[1], b[0], b[1])
        if not (np.array_equal(om, o_s) and np.array_equal(lm, l_s)):
            return False
    om, lm = O.lse_merge(o_e, l_e, o_e, l_e)
    return bool((om == 0).all() and np.isneginf(lm).all())


def test_lse_merge_empty_parts():
    assert _lse_merge_empty_pins_hold()


# ---------------------------------------------------------------------------
# anchor count (Section 5 Default Settings; the workloads print K=13, Top-205)
# ---------------------------------------------------------------------------
def test_anchor_count():
    assert O.anchor_count(64, 0.2) == 13
    assert O.anchor_count(1024, 0.2) == 205
    assert O.anchor_count(2048, 0.2) == 410
    assert O.anchor_count(4096, 0.2) == 820
    assert O.anchor_count(16384, 0.3) == 4916
    assert O.anchor_count(30, 0.1) == 3           # 0.1*30 = 3.0000000000000004 in fp64
    assert O.anchor_count(10, 0.5) == 5
    assert O.anchor_count(777, 0.0) == 0
    assert O.anchor_count(777, 1.0) == 777
    with pytest.raises(ValueError):
        O.anchor_count(10, 1.5)
    with pytest.raises(ValueError):
        O.anchor_count(10, float("nan"))


# ---------------------------------------------------------------------------
# closed forms and invariants of Eq. (4)-(5)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kw", [{}, dict(n_q_heads=4, n_kv_heads=4), dict(dtype="bf16")])
def test_score_total_is_NHm(kw):
    """Each masked row's Eq. (4) weights form a softmax over the affix, so
    sum_j s_j = N * H * m exactly (P1)."""
    w = tiny_workload(**kw)
    K, lay, k, v, q = build_case(w)
    s = O.probe_scores(q, k, v, lay.shared_slots, w.page_size, w.n_kv_heads, lay.masked_rows,
                       lay.masked_offsets, 1 / math.sqrt(w.head_dim))
    tot = w.n_layers * w.n_q_heads * w.m
    np.testing.assert_allclose(s.sum(axis=1), tot, rtol=1e-12)
    assert (s > 0).all()
    # every probe row's weights sum to one: the LSE normalises the row
    _, lse, _ = O.probe_layer(q[0], k[0], v[0], lay.shared_slots, w.page_size, w.n_kv_heads,
                              lay.masked_rows, lay.masked_offsets, 1 / math.sqrt(w.head_dim))
    for h in range(w.n_q_heads):
        g = h // (w.n_q_heads // w.n_kv_heads)
        keys = np.array([O.decode(k[0][s // w.page_size, g, s % w.page_size]) for s in lay.shared_slots])
        S = O.decode(q[0][:, h]) @ keys.T / math.sqrt(w.head_dim)
        np.testing.assert_allclose(np.exp(S - lse[:, h][:, None]).sum(axis=1), 1.0, rtol=1e-12)


def test_uniform_when_q_zero():
    """Q = 0 makes every logit equal: s_j = N H m / L, O_aff is the mean affix
    value, mapped O is the mean of the gathered values (P2)."""
    w = tiny_workload()
    K, lay, k, v, q = build_case(w)
    q = np.zeros_like(q)
    scale = 1 / math.sqrt(w.head_dim)
    s = O.probe_scores(q, k, v, lay.shared_slots, w.page_size, w.n_kv_heads, lay.masked_rows,
                       lay.masked_offsets, scale)
    np.testing.assert_allclose(s, w.n_layers * w.n_q_heads * w.m / w.L, rtol=1e-12)
    o, _, _ = O.probe_layer(q[1], k[1], v[1], lay.shared_slots, w.page_size, w.n_kv_heads,
                            lay.masked_rows, lay.masked_offsets, scale)
    kv = torch.from_numpy(v[1]).double().permute(1, 0, 2, 3).reshape(w.n_kv_heads, -1, w.head_dim)
    mean_aff = kv[:, torch.from_numpy(lay.shared_slots.astype(np.int64))].mean(dim=1).numpy()
    for h in range(w.n_q_heads):
        np.testing.assert_allclose(o[:, h], np.broadcast_to(mean_aff[h // 2], o[:, h].shape), atol=1e-12)
    anchors = [O.topk_anchors(s[b], K, w.affix_l) for b in range(w.batch)]
    read, _, _ = full_maps(w, K, lay, anchors)
    qd = np.zeros((3 * w.batch, w.n_q_heads, w.head_dim))
    om, _ = O.mapped_attention_layer(qd, k[1], v[1], [0, 3, 6], read, lay.kv_offsets, w.n_kv_heads,
                                     w.page_size, scale)
    for b in range(w.batch):
        rs = torch.from_numpy(read[lay.kv_offsets[b]:lay.kv_offsets[b + 1]].astype(np.int64))
        mean_b = kv[:, rs].mean(dim=1).numpy()
        for h in range(w.n_q_heads):
            np.testing.assert_allclose(om[3 * b:3 * b + 3, h], np.broadcast_to(mean_b[h // 2], (3, w.head_dim)),
                                       atol=1e-12)


def test_single_affix_token():
    """L = 1: the lone affix key takes all mass, s = N H m; K = 1 picks it (P3)."""
    w = tiny_workload(segments=(("req", 2), ("affix", 1), ("gen", 3)))
    K, lay, k, v, q = build_case(w, K=1)
    s = O.probe_scores(q, k, v, lay.shared_slots, w.page_size, w.n_kv_heads, lay.masked_rows,
                       lay.masked_offsets, 1 / math.sqrt(w.head_dim))
    np.testing.assert_allclose(s, w.n_layers * w.n_q_heads * w.m, rtol=1e-14)
    assert O.topk_anchors(s[0], 1, w.affix_l).tolist() == [w.affix_l]


def test_dominant_key_takes_all_mass():
    """One affix key whose logit beats every other by > 60 for every query and
    head carries ~N H m of the score and ranks first (P4)."""
    w = tiny_workload()
    K, lay, k, v, q = build_case(w)
    q = np.abs(q)
    q[..., 0] = 1.0
    k = k.copy()
    j = 7
    k[:, :, :, :, :] = np.clip(k, -0.1, 0.1)
    s_j = int(lay.shared_slots[j])
    k[:, s_j // w.page_size, :, s_j % w.page_size, :] = 0.0
    k[:, s_j // w.page_size, :, s_j % w.page_size, 0] = 1000.0
    s = O.probe_scores(q, k, v, lay.shared_slots, w.page_size, w.n_kv_heads, lay.masked_rows,
                       lay.masked_offsets, 1 / math.sqrt(w.head_dim))
    tot = w.n_layers * w.n_q_heads * w.m
    np.testing.assert_allclose(s[:, j], tot, rtol=1e-12)
    others = np.delete(s, j, axis=1)
    assert others.max() < 1e-20 * tot
    for b in range(w.batch):
        assert O.topk_anchors(s[b], 1, w.affix_l).tolist() == [w.affix_l + j]


# ---------------------------------------------------------------------------
# mapped attention: special cases and invariants (Section 4.1, 4.3, App. C.1)
# ---------------------------------------------------------------------------
def _sdpa(q, k, v):
    """torch scaled_dot_product_attention in fp64 on CPU.  q [nq][Hq][d],
    k/v [T][Hkv][d] -> [nq][Hq][d]."""
    Hq, Hkv = q.shape[1], k.shape[1]
    qt = torch.from_numpy(np.ascontiguousarray(q)).double().permute(1, 0, 2)[None]
    kt = torch.from_numpy(np.ascontiguousarray(k)).double().permute(1, 0, 2)[None]
    vt = torch.from_numpy(np.ascontiguousarray(v)).double().permute(1, 0, 2)[None]
    kt = kt.repeat_interleave(Hq // Hkv, dim=1)
    vt = vt.repeat_interleave(Hq // Hkv, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=False)
    return o[0].permute(1, 0, 2).numpy()


def _flat(pool_layer):
    """[n_pages][Hkv][ps][d] -> [slots][Hkv][d] by reshaping (not slot_rows)."""
    t = torch.from_numpy(O.decode(pool_layer))
    return t.permute(0, 2, 1, 3).reshape(-1, t.shape[1], t.shape[3]).numpy()


def test_identity_map_equals_contiguous_sdpa():
    """Rate 0, prefix affix, pages in natural order: the read-slot map is the
    identity and mapped attention is plain attention over pool slots 0..T-1,
    checked against torch's SDPA (P5)."""
    w = tiny_workload(segments=(("affix", 12), ("req", 4), ("gen", 8)), batch=1, page_order="identity", rate=0.0)
    K, lay, k, v, q = build_case(w)
    assert K == 0
    read, _, _ = full_maps(w, K, lay, [O.topk_anchors(np.zeros(w.L), 0, 0)])
    assert read.tolist() == list(range(w.T))
    qd = np_of(gen.make_rows(w, 5, gen.S_QDEC, heads=w.n_q_heads))
    scale = 1 / math.sqrt(w.head_dim)
    for n in range(w.n_layers):
        om, _ = O.mapped_attention_layer(qd[n], k[n], v[n], [0, 5], read, lay.kv_offsets, w.n_kv_heads,
                                         w.page_size, scale)
        ref = _sdpa(O.decode(qd[n]), _flat(k[n])[:w.T], _flat(v[n])[:w.T])
        np.testing.assert_allclose(om, ref, atol=1e-12)


def test_physical_permutation_invariance():
    """Moving K/V rows to other physical slots and remapping the read-slot
    table leaves the output unchanged: attention sees the same logical view
    (P6).  The oracle walks keys in logical order, so equality is exact."""
    w = tiny_workload()
    K, lay, k, v, q = build_case(w)
    scale = 1 / math.sqrt(w.head_dim)
    s = O.probe_scores(q, k, v, lay.shared_slots, w.page_size, w.n_kv_heads, lay.masked_rows,
                       lay.masked_offsets, scale)
    anchors = [O.topk_anchors(s[b], K, w.affix_l) for b in range(w.batch)]
    read, _, _ = full_maps(w, K, lay, anchors)
    qd = np_of(gen.make_rows(w, 2 * w.batch, gen.S_QDEC, heads=w.n_q_heads))
    qoff = [0, 2, 4]
    o1, l1 = O.mapped_attention_layer(qd[0], k[0], v[0], qoff, read, lay.kv_offsets, w.n_kv_heads,
                                      w.page_size, scale)
    nslot = lay.n_pages * w.page_size
    perm = np.random.default_rng(5).permutation(nslot)
    k2 = np.empty_like(k[0]); v2 = np.empty_like(v[0])
    for s0 in range(nslot):
        s1 = perm[s0]
        k2[s1 // w.page_size, :, s1 % w.page_size] = k[0][s0 // w.page_size, :, s0 % w.page_size]
        v2[s1 // w.page_size, :, s1 % w.page_size] = v[0][s0 // w.page_size, :, s0 % w.page_size]
    o2, l2 = O.mapped_attention_layer(qd[0], k2, v2, qoff, perm[read], lay.kv_offsets, w.n_kv_heads,
                                      w.page_size, scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def _logical_kv(w, lay, pool_layer, fresh_rows, read_positions_fresh):
    """Assemble a request's logical K (or V) by hand: affix positions in
    `read_positions_fresh` take the fresh row, other affix positions the
    shared row, non-affix positions the fresh row (rows in ascending position
    order)."""
    flat = _flat(pool_layer)
    fresh_iter = iter(range(len(fresh_rows)))
    out = []
    for p in range(w.T):
        in_affix = w.affix_l <= p < w.affix_l + w.L
        if in_affix and p not in read_positions_fresh:
            out.append(flat[lay.shared_slots[p - w.affix_l]])
        else:
            out.append(O.decode(fresh_rows[next(fresh_iter)]))
    return np.array(out)


@pytest.mark.parametrize("rate", [0.0, 1.0])
def test_rate_zero_and_one(rate):
    """Rate 1 recomputes the whole affix: no read touches the shared region
    and attention runs over [fresh affix + fresh rest] (P7).  Rate 0 is direct
    reuse: attention runs over [shared affix + fresh rest] (P8).  Section 5.1."""
    w = tiny_workload(rate=rate)
    K, lay, k, v, q = build_case(w)
    assert K == (w.L if rate == 1.0 else 0)
    scale = 1 / math.sqrt(w.head_dim)
    s = O.probe_scores(q, k, v, lay.shared_slots, w.page_size, w.n_kv_heads, lay.masked_rows,
                       lay.masked_offsets, scale)
    anchors = [O.topk_anchors(s[b], K, w.affix_l) for b in range(w.batch)]
    read, rcp, rcs = full_maps(w, K, lay, anchors)
    shared = set(lay.shared_slots.tolist())
    n_shared_reads = sum(1 for x in read if int(x) in shared)
    assert n_shared_reads == (0 if rate == 1.0 else w.batch * w.L)
    n_rows = len(rcs)
    sk = np_of(gen.make_rows(w, n_rows, gen.S_SRC_K))
    sv = np_of(gen.make_rows(w, n_rows, gen.S_SRC_V))
    kp, vp = k.copy(), v.copy()
    O.scatter(kp, vp, sk, sv, rcs, w.page_size)
    qd = np_of(gen.make_rows(w, 2 * w.batch, gen.S_QDEC, heads=w.n_q_heads))
    for n in range(w.n_layers):
        om, _ = O.mapped_attention_layer(qd[n], kp[n], vp[n], [0, 2, 4], read, lay.kv_offsets, w.n_kv_heads,
                                         w.page_size, scale)
        for b in range(w.batch):
            r0, r1 = lay.rc_offsets[b], lay.rc_offsets[b + 1]
            fresh_pos = set(int(a) for a in anchors[b])
            Kl = _logical_kv(w, lay, k[n], sk[n, r0:r1], fresh_pos)
            Vl = _logical_kv(w, lay, v[n], sv[n, r0:r1], fresh_pos)
            ref = _sdpa(O.decode(qd[n, 2 * b:2 * b + 2]), Kl, Vl)
            np.testing.assert_allclose(om[2 * b:2 * b + 2], ref, atol=1e-12)


# ---------------------------------------------------------------------------
# Top-K on planted inputs (Eq. 6)
# ---------------------------------------------------------------------------
def test_topk_planted():
    L = 50
    assert O.topk_anchors(np.ones(L), 7, 3).tolist() == list(range(3, 10))       # all equal -> first K
    assert O.topk_anchors(-np.arange(L, dtype=float), 7, 0).tolist() == list(range(7))  # decreasing
    assert O.topk_anchors(np.arange(L, dtype=float), 7, 0).tolist() == list(range(43, 50))  # increasing
    assert O.topk_anchors(np.random.rand(L), 0, 0).tolist() == []
    assert O.topk_anchors(np.random.rand(L), L, 5).tolist() == list(range(5, 55))
    rng = np.random.default_rng(1)
    for _ in range(20):
        s = rng.integers(0, 6, L).astype(float)      # many exact ties at every boundary
        K = int(rng.integers(0, L + 1))
        assert O.topk_anchors(s, K, 2).tolist() == brute.topk(s.tolist(), K, 2)


# ---------------------------------------------------------------------------
# map and scatter properties (Section 4.1, 4.2; Appendix C.1)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("segments", [
    (("affix", 13), ("req", 3), ("gen", 6)),
    (("req", 3), ("affix", 13), ("req", 2), ("gen", 6)),
    (("req", 3), ("gen", 6), ("affix", 13)),
])
def test_table_properties(segments):
    w = tiny_workload(segments=segments, page_size=4)
    K, lay, k, v, q = build_case(w)
    rng = np.random.default_rng(3)
    anchors = [np.sort(rng.choice(w.L, K, replace=False)) + w.affix_l for _ in range(w.batch)]
    read, rcp, rcs = full_maps(w, K, lay, anchors)
    shared = lay.shared_slots.tolist()
    for b in range(w.batch):
        rd = read[lay.kv_offsets[b]:lay.kv_offsets[b + 1]]
        assert len(rd) == w.T and (rd >= 0).all()
        A = set(int(a) for a in anchors[b])
        F = set(range(w.affix_l, w.affix_l + w.L))
        for p in range(w.T):
            if p in F and p not in A:
                assert rd[p] == shared[p - w.affix_l]
            else:
                assert rd[p] not in shared
        pp = lay.private_pages[lay.private_page_offsets[b]:lay.private_page_offsets[b + 1]]
        first_R = [int(pp[i // w.page_size]) * w.page_size + i % w.page_size for i in range(K + w.P)]
        ps_ = rcs[lay.rc_offsets[b]:lay.rc_offsets[b + 1]]
        assert sorted(ps_.tolist()) == sorted(first_R) and len(set(ps_.tolist())) == K + w.P
        assert rcp[lay.rc_offsets[b]:lay.rc_offsets[b + 1]].tolist() == sorted(A | (set(range(w.T)) - F))
        br, bp, bs = brute.maps(anchors[b], w.T, w.affix_l, w.L, shared, pp, w.page_size)
        assert br == rd.tolist() and bp == rcp[lay.rc_offsets[b]:lay.rc_offsets[b + 1]].tolist()
        assert bs == ps_.tolist()


def test_scatter_properties():
    w = tiny_workload(dtype="bf16")
    K, lay, k, v, q = build_case(w)
    rng = np.random.default_rng(4)
    anchors = [np.sort(rng.choice(w.L, K, replace=False)) + w.affix_l for _ in range(w.batch)]
    _, _, rcs = full_maps(w, K, lay, anchors)
    sk = np_of(gen.make_rows(w, len(rcs), gen.S_SRC_K))
    sv = np_of(gen.make_rows(w, len(rcs), gen.S_SRC_V))
    kp, vp = k.copy(), v.copy()
    O.scatter(kp, vp, sk, sv, rcs, w.page_size)
    written = np.zeros((lay.n_pages, w.page_size), bool)
    for i, s in enumerate(rcs):
        written[s // w.page_size, s % w.page_size] = True
        assert np.array_equal(kp[:, s // w.page_size, :, s % w.page_size], sk[:, i])
        assert np.array_equal(vp[:, s // w.page_size, :, s % w.page_size], sv[:, i])
    mask = ~written
    assert np.array_equal(kp[:, mask.nonzero()[0], :, mask.nonzero()[1]], k[:, mask.nonzero()[0], :, mask.nonzero()[1]])
    assert np.array_equal(vp.transpose(0, 1, 3, 2, 4)[:, mask], v.transpose(0, 1, 3, 2, 4)[:, mask])
    sh = lay.page_owner == -1
    assert np.array_equal(kp[:, sh], k[:, sh]) and np.array_equal(vp[:, sh], v[:, sh])
    kp2, vp2 = kp.copy(), vp.copy()
    O.scatter(kp2, vp2, sk, sv, rcs, w.page_size)
    assert np.array_equal(kp2, kp) and np.array_equal(vp2, vp)


# ---------------------------------------------------------------------------
# brute force (pure Python loops) against the oracle (P12)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("wl,order", [
    (WORKLOADS[1], "identity"),
    (WORKLOADS[1].scaled(shared_slot_order="slot", page_order="random"), "random"),
    (tiny_workload(), "random"),
    (tiny_workload(dtype="bf16", n_q_heads=6, n_kv_heads=2,
                   segments=(("req", 2), ("gen", 4), ("affix", 9))), "fragmented"),
])
def test_brute_force_agrees(wl, order):
    w = wl.scaled(page_order=order, free_frac=0.25 if order == "fragmented" else 0.0)
    K, lay, k, v, q = build_case(w)
    scale = 1 / math.sqrt(w.head_dim)
    o_s = np.zeros((w.batch, w.L))
    o_aff = []
    for n in range(w.n_layers):
        o, lse, s = O.probe_layer(q[n], k[n], v[n], lay.shared_slots, w.page_size, w.n_kv_heads,
                                  lay.masked_rows, lay.masked_offsets, scale)
        o_s += s
        o_aff.append(o)
    b_s, b_o, _ = brute.probe(q, k, v, lay.shared_slots, w.page_size, w.n_kv_heads, lay.masked_rows,
                              lay.masked_offsets, scale)
    np.testing.assert_allclose(o_s, np.array(b_s), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(np.array(o_aff), np.array(b_o), atol=1e-12)
    anchors = [O.topk_anchors(o_s[b], K, w.affix_l) for b in range(w.batch)]
    for b in range(w.batch):
        assert anchors[b].tolist() == brute.topk(b_s[b], K, w.affix_l)
    read, _, _ = full_maps(w, K, lay, anchors)
    nq = 3
    qd = np_of(gen.make_rows(w, nq * w.batch, gen.S_QDEC, heads=w.n_q_heads))
    qoff = list(range(0, nq * w.batch + 1, nq))
    om = [O.mapped_attention_layer(qd[n], k[n], v[n], qoff, read, lay.kv_offsets, w.n_kv_heads, w.page_size,
                                   scale)[0] for n in range(w.n_layers)]
    bo = brute.mapped_attention(qd, k, v, qoff, read, lay.kv_offsets, w.n_kv_heads, w.page_size, scale)
    np.testing.assert_allclose(np.array(om), np.array(bo), atol=1e-12)


# ---------------------------------------------------------------------------
# the pins catch planted mistakes in the oracle
# ---------------------------------------------------------------------------
def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible slips in the oracle and check a pin fails for each:
    a wrong GQA head mapping, masked-row sums taken over every row, ties
    broken toward the higher offset, decode-block slots read without the
    request's table offset or with a wrong block range, an LSE merge
    without its empty-part branch."""
    w = tiny_workload()
    K, lay, k, v, q = build_case(w)
    scale = 1 / math.sqrt(w.head_dim)

    def brute_gap():
        s = O.probe_scores(q, k, v, lay.shared_slots, w.page_size, w.n_kv_heads, lay.masked_rows,
                           lay.masked_offsets, scale)
        b_s, _, _ = brute.probe(q, k, v, lay.shared_slots, w.page_size, w.n_kv_heads, lay.masked_rows,
                                lay.masked_offsets, scale)
        return np.abs(s - np.array(b_s)).max()

    assert brute_gap() < 1e-12
    with monkeypatch.context() as m:
        m.setattr(O, "kv_head_of", lambda h, hq, hkv: h % hkv)
        assert brute_gap() > 1e-6
    all_rows = np.arange(q.shape[1], dtype=np.int32)
    s_bad = O.probe_scores(q, k, v, lay.shared_slots, w.page_size, w.n_kv_heads, all_rows,
                           np.array([0, len(all_rows) // 2, len(all_rows)]), scale)
    assert abs(s_bad.sum(axis=1)[0] - w.n_layers * w.n_q_heads * w.m) > 1.0
    g = gold("topk_ties.json")
    with monkeypatch.context() as m:
        m.setattr(O, "topk_anchors",
                  lambda sc, kk, l: np.sort(np.lexsort((-np.arange(len(sc)), -np.asarray(sc)))[:kk]) + l)
        assert O.topk_anchors(np.array(g["scores"]), 5, g["affix_l"]).tolist() != g["cases"]["5"]
    # decode-block slots read without the request's table offset
    assert _block_slots_pins_hold()
    with monkeypatch.context() as m:
        m.setattr(O, "block_slots", lambda rs, ko, bs, bl: np.array(
            [int(rs[bs[b] + i]) for b in range(len(ko) - 1) for i in range(bl)], np.int64))
        assert not _block_slots_pins_hold()
    # ... or with the block's length taken as its end position
    with monkeypatch.context() as m:
        m.setattr(O, "block_slots", lambda rs, ko, bs, bl: np.array(
            [int(rs[ko[b] + i]) for b in range(len(ko) - 1) for i in range(bs[b], bl)], np.int64))
        assert not _block_slots_pins_hold()
    # an LSE merge without the empty-part branch (weights exp(lse_a - lse) with lse = -inf)
    assert _lse_merge_empty_pins_hold()
    with monkeypatch.context() as m:
        def merge_unguarded(o_a, lse_a, o_b, lse_b):
            lse = np.logaddexp(lse_a, lse_b)
            with np.errstate(invalid="ignore"):
                return (np.exp(lse_a - lse)[..., None] * o_a + np.exp(lse_b - lse)[..., None] * o_b, lse)
        m.setattr(O, "lse_merge", merge_unguarded)
        assert not _lse_merge_empty_pins_hold()


def test_empty_context_is_empty_sum():
    """A request with no logical positions: the attention sum is empty, so
    O = 0 and LSE = log(0) = -inf; other requests are unaffected."""
    w = tiny_workload()
    K, lay, k, v, q = build_case(w)
    qd = np_of(gen.make_rows(w, 4, gen.S_QDEC, heads=w.n_q_heads))
    read = lay.shared_slots[:5]
    o, lse = O.mapped_attention_layer(qd[0], k[0], v[0], [0, 2, 4], read, [0, 0, 5], w.n_kv_heads, w.page_size,
                                      1 / math.sqrt(w.head_dim))
    assert (o[:2] == 0).all() and np.isneginf(lse[:2]).all()
    o2, _ = O.mapped_attention_layer(qd[0][2:], k[0], v[0], [0, 2], read, [0, 5], w.n_kv_heads, w.page_size,
                                     1 / math.sqrt(w.head_dim))
    assert np.array_equal(o[2:], o2)


# ---------------------------------------------------------------------------
# DropNA (Section 5.3, Figure 5) and the KV footprint (Section 4.1, App. B.2)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("rate", [0.0, 0.3, 1.0])
def test_dropna_table_and_attention(rate):
    """DropNA keeps the same anchors and drops the non-anchor affix cache: its
    read list is the KeepNA list minus F \\ A (T - L + K entries), it equals
    the KeepNA list at ratio 1 (no non-anchor tokens remain), and attention
    over it equals attention over the full logical context with the dropped
    positions masked out (torch SDPA with a boolean mask, fp64)."""
    w = tiny_workload(rate=rate)
    K, lay, k, v, q = build_case(w)
    scale = 1 / math.sqrt(w.head_dim)
    s = O.probe_scores(q, k, v, lay.shared_slots, w.page_size, w.n_kv_heads, lay.masked_rows,
                       lay.masked_offsets, scale)
    anchors = [O.topk_anchors(s[b], K, w.affix_l) for b in range(w.batch)]
    read, rcp, rcs = full_maps(w, K, lay, anchors)
    n_rows = len(rcs)
    sk = np_of(gen.make_rows(w, n_rows, gen.S_SRC_K))
    sv = np_of(gen.make_rows(w, n_rows, gen.S_SRC_V))
    kp, vp = k.copy(), v.copy()
    O.scatter(kp, vp, sk, sv, rcs, w.page_size)
    qd = np_of(gen.make_rows(w, 2 * w.batch, gen.S_QDEC, heads=w.n_q_heads))
    for b in range(w.batch):
        T = int(lay.seq_len[b])
        rb = read[lay.kv_offsets[b]:lay.kv_offsets[b + 1]]
        dn = O.dropna_read_table(rb, anchors[b], w.affix_l, w.L)
        assert len(dn) == T - w.L + K
        if rate == 1.0:
            assert dn.tolist() == rb.tolist()
        for n in range(w.n_layers):
            om, _ = O.mapped_attention_layer(qd[n, 2 * b:2 * b + 2], kp[n], vp[n], [0, 2], dn, [0, len(dn)],
                                             w.n_kv_heads, w.page_size, scale)
            fresh_pos = set(int(a) for a in anchors[b])
            r0, r1 = lay.rc_offsets[b], lay.rc_offsets[b + 1]
            Kl = torch.from_numpy(_logical_kv(w, lay, k[n], sk[n, r0:r1], fresh_pos))
            Vl = torch.from_numpy(_logical_kv(w, lay, v[n], sv[n, r0:r1], fresh_pos))
            keep = torch.tensor([not (w.affix_l <= p < w.affix_l + w.L) or p in fresh_pos for p in range(T)])
            qq = torch.from_numpy(O.decode(qd[n, 2 * b:2 * b + 2]))       # [2][Hq][d]
            g = w.n_q_heads // w.n_kv_heads
            Kh = Kl.permute(1, 0, 2).repeat_interleave(g, 0)                 # [Hq][T][d]
            Vh = Vl.permute(1, 0, 2).repeat_interleave(g, 0)
            ref = torch.nn.functional.scaled_dot_product_attention(qq.permute(1, 0, 2), Kh, Vh, attn_mask=keep)
            np.testing.assert_allclose(om, ref.permute(1, 0, 2).numpy(), atol=1e-12)


def test_kv_footprint_closed_form_and_layout_count():
    """The footprint counts the pages a layout actually holds: the distinct
    pages of the shared slots plus each request's private pages (counted from
    the tables built for it), and the dense baseline's whole-context pages."""
    for segments, rate, B in [((("affix", 37), ("req", 5), ("gen", 9)), 0.3, 3),
                              ((("req", 6), ("affix", 64), ("gen", 16)), 0.2, 5),
                              ((("req", 2), ("gen", 7), ("affix", 20)), 1.0, 2)]:
        w = tiny_workload(segments=segments, rate=rate, batch=B)
        K = O.anchor_count(w.L, w.rate)
        lay = gen.make_layout(w, K, 3)
        anchors = [np.arange(w.affix_l, w.affix_l + K)] * B
        read, rcp, rcs = full_maps(w, K, lay, anchors)
        slot_bytes = 7
        f = O.kv_footprint(lay.seq_len.tolist(), w.L, K, w.page_size, slot_bytes)
        pages = lambda slots: len(set(int(x) // w.page_size for x in slots))
        assert f["shared"] == pages(lay.shared_slots) * w.page_size * slot_bytes
        priv = sum(pages(rcs[lay.rc_offsets[b]:lay.rc_offsets[b + 1]]) for b in range(B))
        assert f["private"] == priv * w.page_size * slot_bytes
        assert f["dense"] == sum(-(-int(t) // w.page_size) for t in lay.seq_len) * w.page_size * slot_bytes
        assert f["acache"] == f["shared"] + f["private"] and f["dropna"] == f["private"]


def test_kv_footprint_hand_numbers_and_trend():
    """LLaDA-8B shapes (32 layers, 32 KV heads, d=128, bf16: 512 KiB of K and V
    per slot), 16-slot pages, affix 4096, 512 request positions, K = 820:
    dense 16 * 288 pages, ACache 256 + 16 * 84 pages.  Appendix B.2: at batch
    1 the separate shared and private blocks cost at least the dense cache,
    and the saving grows with the batch."""
    sb = 32 * 32 * 128 * 2 * 2
    f = O.kv_footprint([4608] * 16, 4096, 820, 16, sb)
    assert f["dense"] == 16 * 288 * 16 * sb == 38654705664
    assert f["acache"] == (256 + 16 * 84) * 16 * sb == 13421772800
    one = O.kv_footprint([4608], 4096, 820, 16, sb)
    assert one["acache"] >= one["dense"]
    red = [1 - O.kv_footprint([4608] * B, 4096, 820, 16, sb)["acache"] / (B * 288 * 16 * sb) for B in (1, 2, 4, 16)]
    assert red == sorted(red) and red[-1] > 0.6


# ---------------------------------------------------------------------------
# full-context normaliser of the probe (the alternative reading of Eq. (4))
# ---------------------------------------------------------------------------
def _na_slots(w, lay):
    """Slots for each request's non-affix keys: the first P_b slots of its
    private pages (any valid slots serve; the pool is random there)."""
    out, offs = [], [0]
    for b in range(w.batch):
        pp = lay.private_pages[lay.private_page_offsets[b]:lay.private_page_offsets[b + 1]]
        P_b = int(lay.row_offsets[b + 1] - lay.row_offsets[b])
        out += [int(pp[i // w.page_size]) * w.page_size + i % w.page_size for i in range(P_b)]
        offs.append(len(out))
    return np.array(out, np.int64), np.array(offs, np.int64)


def test_probe_full_normaliser_pins():
    """(i) O and LSE equal torch SDPA / logsumexp over [affix keys, own
    non-affix keys] (fp64); (ii) the affix weights under the full normaliser
    are the affix-only weights times exp(LSE_aff - LSE_all), summed over the
    masked rows; (iii) merging the affix-only attention with the attention
    over the own keys gives the same O and LSE; (iv) with no own keys the
    full normaliser is the affix-only one."""
    w = tiny_workload(segments=(("req", 3), ("affix", 11), ("req", 2), ("gen", 5)), batch=2)
    K, lay, k, v, q = build_case(w)
    scale = 1 / math.sqrt(w.head_dim)
    na, na_off = _na_slots(w, lay)
    for n in range(w.n_layers):
        of, lf, sf = O.probe_layer_full(q[n], k[n], v[n], lay.shared_slots, lay.row_offsets, na, na_off, w.page_size,
                                        w.n_kv_heads, lay.masked_rows, lay.masked_offsets, scale)
        oa, la, _ = O.probe_layer(q[n], k[n], v[n], lay.shared_slots, w.page_size, w.n_kv_heads, lay.masked_rows,
                                  lay.masked_offsets, scale)
        on, ln = O.mapped_attention_layer(q[n], k[n], v[n], lay.row_offsets, na, na_off, w.n_kv_heads, w.page_size,
                                          scale)
        om, lm = O.lse_merge(oa, la, on, ln)
        np.testing.assert_allclose(om, of, atol=1e-12)
        np.testing.assert_allclose(lm, lf, atol=1e-12)
        sref = np.zeros_like(sf)
        for b in range(w.batch):
            r0, r1 = lay.row_offsets[b], lay.row_offsets[b + 1]
            own = na[na_off[b]:na_off[b + 1]]
            for h in range(w.n_q_heads):
                g = h // (w.n_q_heads // w.n_kv_heads)
                kk = torch.from_numpy(np.concatenate([O.slot_rows(k[n], lay.shared_slots, g, w.page_size),
                                                      O.slot_rows(k[n], own, g, w.page_size)]))
                vv = torch.from_numpy(np.concatenate([O.slot_rows(v[n], lay.shared_slots, g, w.page_size),
                                                      O.slot_rows(v[n], own, g, w.page_size)]))
                qq = torch.from_numpy(O.decode(q[n, r0:r1, h, :]))
                ref = torch.nn.functional.scaled_dot_product_attention(qq[None], kk[None], vv[None])[0]
                np.testing.assert_allclose(of[r0:r1, h], ref.numpy(), atol=1e-12)
                lall = torch.logsumexp((qq @ kk.T) * scale, dim=1).numpy()
                np.testing.assert_allclose(lf[r0:r1, h], lall, atol=1e-12)
                aff = torch.softmax((qq @ kk[:w.L].T) * scale, dim=1).numpy()        # affix-only weights
                mk = lay.masked_rows[lay.masked_offsets[b]:lay.masked_offsets[b + 1]] - r0
                sref[b] += (aff[mk] * np.exp(la[r0:r1, h][mk] - lall[mk])[:, None]).sum(axis=0)
        np.testing.assert_allclose(sf, sref, rtol=1e-10, atol=1e-14)
        assert (sf.sum(axis=1) < w.n_q_heads * np.diff(lay.masked_offsets)).all()
        o0, l0, s0 = O.probe_layer_full(q[n], k[n], v[n], lay.shared_slots, lay.row_offsets, na[:0],
                                        np.zeros(w.batch + 1, np.int64), w.page_size, w.n_kv_heads,
                                        lay.masked_rows, lay.masked_offsets, scale)
        _, _, sa = O.probe_layer(q[n], k[n], v[n], lay.shared_slots, w.page_size, w.n_kv_heads, lay.masked_rows,
                                 lay.masked_offsets, scale)
        np.testing.assert_allclose(o0, oa, atol=1e-12)
        np.testing.assert_allclose(l0, la, atol=1e-12)
        np.testing.assert_allclose(s0, sa, atol=1e-12)


# ---------------------------------------------------------------------------
# HKVD selector (Appendix B.5)
# ---------------------------------------------------------------------------
def test_hkvd_scores_pins():
    """Zero for a full-prompt cache identical to the shared one; a planted
    deviation of c on one element of one token adds exactly c^2 there; in
    general the torch vector norm of the token's whole KV difference,
    squared."""
    w = tiny_workload(dtype="f32", segments=(("affix", 20), ("req", 4), ("gen", 4)), batch=3)
    K, lay, k, v, q = build_case(w)
    N, Hkv, d, L, B = w.n_layers, w.n_kv_heads, w.head_dim, w.L, w.batch
    same_k = np.stack([np.stack([np.stack([O.slot_rows(k[n], lay.shared_slots, g, w.page_size) for g in range(Hkv)], 1)
                                 for _ in range(B)]) for n in range(N)])
    same_v = np.stack([np.stack([np.stack([O.slot_rows(v[n], lay.shared_slots, g, w.page_size) for g in range(Hkv)], 1)
                                 for _ in range(B)]) for n in range(N)])
    assert same_k.shape == (N, B, L, Hkv, d)
    assert (O.hkvd_scores(k, v, lay.shared_slots, same_k, same_v, w.page_size) == 0).all()
    pk = same_k.copy()
    pk[1, 2, 7, 1, 3] += 0.5
    s = O.hkvd_scores(k, v, lay.shared_slots, pk, same_v, w.page_size)
    assert s[2, 7] == 0.25 and s.sum() == 0.25
    rng = np.random.default_rng(5)
    fk = rng.standard_normal(same_k.shape)
    fv = rng.standard_normal(same_v.shape)
    s = O.hkvd_scores(k, v, lay.shared_slots, fk, fv, w.page_size)
    for b in range(B):
        for j in range(L):
            diff = np.concatenate([(fk[:, b, j] - same_k[:, b, j]).ravel(), (fv[:, b, j] - same_v[:, b, j]).ravel()])
            assert abs(s[b, j] - torch.linalg.vector_norm(torch.from_numpy(diff)).item() ** 2) <= 1e-9 * s[b, j]
