"""GPU parity: the library (through its C ABI) against the fp64 oracle on the
same seeded inputs.  Stage by stage: probe scores, O_aff and LSE (Eq. 4-5),
anchor sets (Eq. 6), both maps (Section 4.1-4.2), the private scatter and the
read-slot attention (Section 4.3, Appendix C.1)."""
import math

import numpy as np
import pytest
import torch

import attention_anchor_probe_amd as A
from oracle import acache_oracle as O
from synth.configs import WORKLOADS, Workload
from synth import gen
from tests.gpu_common import DEV, Chain, anchors_match, bf16_close, i32
from tests.helpers import np_of

pytestmark = pytest.mark.gpu


def _check_chain(c, layers, fp32):
    w = c.w
    s_gpu = c.scores.cpu().numpy().astype(np.float64)
    big = c.r_scores >= 1e-6 * c.r_scores.max()
    rel = np.abs(s_gpu - c.r_scores)[big] / c.r_scores[big]
    assert rel.max() <= (1e-5 if fp32 else 1e-3), f"scores rel err {rel.max()}"
    assert np.abs(s_gpu - c.r_scores)[~big].max(initial=0) <= 1e-9 * c.r_scores.sum()
    tot = w.n_layers * w.n_q_heads * w.m
    np.testing.assert_allclose(s_gpu.sum(axis=1), tot, rtol=1e-4)
    an = c.anchors.cpu().numpy()
    exact_all = True
    for b in range(w.batch):
        ok, exact = anchors_match(c.r_scores[b], an[b], c.K, w.affix_l)
        assert ok, f"anchor set of request {b} differs beyond the tie band"
        exact_all &= exact
        # the kernel's Top-K on its own fp32 scores equals the sort-based Top-K of those scores
        assert an[b].tolist() == O.topk_anchors(s_gpu[b], c.K, w.affix_l).tolist()
    for n in layers:
        oa = np_of(c.o_aff[n]).astype(np.float64) if fp32 else c.o_aff[n].float().cpu().numpy()
        if fp32:
            assert np.abs(oa - c.r_oaff[n]).max() <= 1e-5
        else:
            ok, st = bf16_close(oa, c.r_oaff[n])
            assert ok, f"O_aff layer {n}: {st}"
        np.testing.assert_allclose(c.lse_aff[n].cpu().numpy(), c.r_lseaff[n], atol=1e-4 if not fp32 else 1e-5)
    if not exact_all:
        # the sets differ only inside the tie band (checked above): the oracle's
        # maps, scatter and attention are taken from the library's anchors
        c.run_oracle_downstream(list(an), c.r_layers)
    assert np.array_equal(c.read_slot.cpu().numpy(), c.r_read)
    assert np.array_equal(c.rc_pos.cpu().numpy(), c.r_rcpos)
    assert np.array_equal(c.rc_slot.cpu().numpy(), c.r_rcslot)
    kpool, vpool = np_of(c.k), np_of(c.v)
    for i, n in enumerate(c.r_layers):
        assert np.array_equal(kpool[n], c.r_kpool[i]) and np.array_equal(vpool[n], c.r_vpool[i])
        for tag, out, lse in (("", c.out, c.lse), ("shared-affix ", c.out_sh, c.lse_sh)):
            o = np_of(out[n]).astype(np.float64) if fp32 else out[n].float().cpu().numpy()
            if fp32:
                assert np.abs(o - c.r_out[n]).max() <= 1e-5
            else:
                ok, st = bf16_close(o, c.r_out[n])
                assert ok, f"{tag}mapped attention layer {n}: {st}"
            np.testing.assert_allclose(lse[n].cpu().numpy(), c.r_lse[n], atol=1e-4)


@pytest.mark.parametrize("order,slot_order", [("identity", "page"), ("random", "slot")])
def test_tiny_fp32_full_chain(order, slot_order):
    """The tiny fp32 workload (1 layer, 2 heads, d=16, L=64, K=13), with the
    identity and a randomly permuted slot layout."""
    w = WORKLOADS[1]
    c = Chain(w, page_order=order, shared_slot_order=slot_order)
    if order == "identity":
        assert c.lay.shared_slots.tolist() == list(range(64))
    c.run_gpu()
    c.run_oracle()
    _check_chain(c, [0], fp32=True)


SMALL = [
    # (name, workload) small shapes spanning several tiles and ragged tails
    ("bf16-d64-prefix", Workload(91, "s1", "bf16", 2, 4, 4, 64, (("affix", 200), ("req", 24), ("gen", 40)), 2, 0.2,
                                 page_order="random")),
    ("bf16-d128-infix-gqa", Workload(92, "s2", "bf16", 2, 8, 2, 128,
                                     (("req", 9), ("affix", 300), ("req", 7), ("gen", 64)), 3, 0.2,
                                     page_order="random", key_tweak="sinks")),
    ("bf16-d128-suffix", Workload(93, "s3", "bf16", 2, 4, 4, 128, (("req", 33), ("gen", 64), ("affix", 257)), 2, 0.3,
                                  page_order="fragmented", free_frac=0.125, key_tweak="heavy")),
    ("f32-d32-prefix", Workload(94, "s4", "f32", 2, 4, 2, 32, (("affix", 70), ("req", 5), ("gen", 37)), 2, 0.5,
                                page_order="random")),
    ("bf16-d16-ps4", Workload(95, "s5", "bf16", 1, 2, 1, 16, (("affix", 45), ("req", 3), ("gen", 19)), 2, 0.2,
                              page_size=4, page_order="random")),
    # large pages: a page holds many slots of every KV head
    ("bf16-d128-ps64", Workload(96, "s6", "bf16", 2, 4, 4, 128, (("affix", 333), ("req", 20), ("gen", 48)), 3, 0.2,
                                page_size=64, page_order="random")),
    ("bf16-d128-ps256-gqa", Workload(97, "s7", "bf16", 1, 8, 2, 128, (("req", 11), ("affix", 600), ("gen", 70)), 2,
                                     0.25, page_size=256, page_order="fragmented", free_frac=0.125)),
    # sixteen query heads per KV head: the probe's packed units hold 16 heads' rows
    ("bf16-d128-g16", Workload(98, "s8", "bf16", 1, 32, 2, 128, (("affix", 200), ("req", 12), ("gen", 40)), 2, 0.2,
                               page_order="random")),
]


@pytest.mark.parametrize("name,w", SMALL, ids=[s[0] for s in SMALL])
def test_small_full_chain(name, w):
    c = Chain(w, n_dec=min(w.block_len, w.m))
    c.run_gpu()
    c.run_oracle()
    _check_chain(c, list(range(w.n_layers)), fp32=w.dtype == "f32")


# ---------------------------------------------------------------------------
# Top-K on seeded scores: bit-exact against the sort-based oracle
# ---------------------------------------------------------------------------
def _topk_case(scores_np, K, affix_l):
    s = torch.as_tensor(scores_np.astype(np.float32), device=DEV)
    B, L = s.shape
    an = torch.full((B, max(K, 1)), -7, dtype=torch.int32, device=DEV)
    A.acache_topk_anchors(s, K, affix_l, an[:, :K] if K > 0 else an[:, :0])
    got = an.cpu().numpy()
    s32 = s.cpu().numpy().astype(np.float64)
    for b in range(B):
        assert got[b, :K].tolist() == O.topk_anchors(s32[b], K, affix_l).tolist(), (b, K)


@pytest.mark.parametrize("L", [1, 5, 64, 1000, 1024, 1025, 4096, 16384, 32768])
def test_topk_seeded(L):
    rng = np.random.default_rng(L)
    B = 3
    s = rng.random((B, L)).astype(np.float32)
    for K in sorted({0, 1, L // 5, (L + 1) // 2, L - 1, L} - {-1}):
        if K < 0:
            continue
        _topk_case(s, K, 7)


def test_topk_ties_and_special_values():
    rng = np.random.default_rng(9)
    L = 3000
    ties = rng.integers(0, 5, (2, L)).astype(np.float32)          # heavy exact ties at every boundary
    for K in (1, 17, 600, 1500, 2999):
        _topk_case(ties, K, 0)
    _topk_case(np.ones((1, L), np.float32), 100, 3)                  # all equal -> first K
    special = rng.standard_normal((1, 257)).astype(np.float32)
    special[0, [3, 50, 51]] = np.nan
    special[0, [4, 5]] = [0.0, -0.0]
    special[0, [6, 7]] = [np.inf, -np.inf]
    special[0, 100:110] = -0.0
    special[0, 110:120] = 0.0
    for K in (1, 2, 100, 250, 254, 255, 257):
        _topk_case(special, K, 0)


# ---------------------------------------------------------------------------
# maps from seeded anchor sets; block slots
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("segments", [
    (("affix", 131), ("req", 17), ("gen", 40)),
    (("req", 9), ("affix", 131), ("req", 5), ("gen", 40)),
    (("req", 9), ("gen", 40), ("affix", 131)),
])
@pytest.mark.parametrize("rate", [0.0, 0.2, 1.0])
def test_maps_seeded(segments, rate):
    w = Workload(96, "maps", "bf16", 1, 2, 2, 16, segments, 5, rate, page_size=8, page_order="fragmented",
                 free_frac=0.2)
    K = A.acache_anchor_count(w.L, rate)
    lay = gen.make_layout(w, K, 3)
    rng = np.random.default_rng(11)
    anchors = np.stack([np.sort(rng.choice(w.L, K, replace=False)) + w.affix_l for _ in range(w.batch)]) \
        if K > 0 else np.zeros((w.batch, 0), np.int64)
    read = torch.empty(int(lay.kv_offsets[-1]), dtype=torch.int32, device=DEV)
    rcp = torch.empty(int(lay.rc_offsets[-1]), dtype=torch.int32, device=DEV)
    rcs = torch.empty_like(rcp)
    keep = [i32(x) for x in (lay.seq_len, lay.shared_slots, lay.private_pages, lay.private_page_offsets,
                             lay.kv_offsets, lay.rc_offsets)]
    maps = A.map_args(w.batch, w.affix_l, w.L, K, w.page_size, w.T, *keep, read, rcp, rcs)
    an_d = i32(anchors.reshape(w.batch, K)) if K > 0 else torch.zeros((w.batch, 0), dtype=torch.int32, device=DEV)
    A.acache_build_maps(an_d, maps)
    torch.cuda.synchronize()
    rd, rp, rs = [], [], []
    for b in range(w.batch):
        pp = lay.private_pages[lay.private_page_offsets[b]:lay.private_page_offsets[b + 1]]
        r_, p_, s_ = O.build_maps(anchors[b], w.T, w.affix_l, w.L, lay.shared_slots, pp, w.page_size)
        rd.append(r_); rp.append(p_); rs.append(s_)
    assert np.array_equal(read.cpu().numpy(), np.concatenate(rd))
    assert np.array_equal(rcp.cpu().numpy(), np.concatenate(rp))
    assert np.array_equal(rcs.cpu().numpy(), np.concatenate(rs))
    # decode-block destination slots read through the map
    bs = np.full(w.batch, w.gen_start(), np.int32)
    dst = torch.empty(w.batch * 16, dtype=torch.int32, device=DEV)
    A.acache_block_slots(read, keep[4], i32(bs), 16, dst)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), O.block_slots(np.concatenate(rd), lay.kv_offsets, bs, 16))


# ---------------------------------------------------------------------------
# scatter on seeded destinations: bit-exact, nothing else touched
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,d,hkv", [("bf16", 128, 4), ("f32", 16, 2), ("bf16", 64, 3)])
def test_scatter_seeded(dtype, d, hkv):
    w = Workload(97, "sc", dtype, 3, hkv, hkv, d, (("affix", 64), ("req", 40), ("gen", 40)), 2, 0.25,
                 page_order="random")
    K = A.acache_anchor_count(w.L, w.rate)
    lay = gen.make_layout(w, K, 1)
    k, v = gen.make_pool(w, lay, device=DEV)
    priv = np.concatenate([(p * w.page_size + np.arange(w.page_size)) for p in lay.private_pages])
    rng = np.random.default_rng(2)
    dst = rng.permutation(priv)[:101].astype(np.int32)
    assert A.acache_validate_slots(dst, lay.page_owner, lay.n_pages, w.page_size)[0] == 0
    sk = gen.make_rows(w, len(dst), gen.S_SRC_K, device=DEV, layers=[1, 2])
    sv = gen.make_rows(w, len(dst), gen.S_SRC_V, device=DEV, layers=[1, 2])
    torch.cuda.synchronize()
    kh, vh, skh, svh = map(np_of, (k, v, sk, sv))
    A.acache_scatter_private(k, v, sk, sv, i32(dst), layer_begin=1)
    torch.cuda.synchronize()
    kr, vr = kh.copy(), vh.copy()
    O.scatter(kr[1:], vr[1:], skh, svh, dst, w.page_size)
    assert np.array_equal(np_of(k), kr) and np.array_equal(np_of(v), vr)
    # zero rows is a no-op
    A.acache_scatter_private(k, v, sk[:, :0], sv[:, :0], i32(dst[:0]), layer_begin=1)
    torch.cuda.synchronize()
    assert np.array_equal(np_of(k), kr)


# ---------------------------------------------------------------------------
# mapped attention edge cases on seeded tables
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 16), ("bf16", 64)])
def test_mapped_attention_ragged(dtype, d):
    """Ragged queries and keys, including a request with no queries, one with
    a single key, one with an empty context (O = 0, LSE = -inf), and query
    counts across several tiles."""
    w = Workload(98, "rag", dtype, 2, 8, 2, d, (("affix", 64), ("req", 8), ("gen", 8)), 5, 0.2, page_order="random")
    K = A.acache_anchor_count(w.L, w.rate)
    lay = gen.make_layout(w, K, 4)
    k, v = gen.make_pool(w, lay, device=DEV)
    nslot = lay.n_pages * w.page_size
    rng = np.random.default_rng(6)
    q_counts = [33, 0, 5, 130, 1]
    kv_counts = [700, 13, 1, 333, 0]
    read = np.concatenate([rng.integers(0, nslot, c) for c in kv_counts]).astype(np.int32)
    q_off = np.concatenate([[0], np.cumsum(q_counts)]).astype(np.int32)
    kv_off = np.concatenate([[0], np.cumsum(kv_counts)]).astype(np.int32)
    qd = gen.make_rows(w, int(q_off[-1]), gen.S_QDEC, device=DEV, heads=w.n_q_heads)
    torch.cuda.synchronize()
    kh, vh, qh = np_of(k), np_of(v), np_of(qd)
    out = torch.full_like(qd, 7.0)
    lse = torch.empty(qd.shape[:3], device=DEV)
    A.acache_mapped_attention(k, v, qd, i32(q_off), i32(read), i32(kv_off), out, lse=lse,
                              max_q_per_req=max(q_counts), max_kv_per_req=max(kv_counts))
    torch.cuda.synchronize()
    for n in range(w.n_layers):
        ref, rl = O.mapped_attention_layer(qh[n], kh[n], vh[n], q_off, read, kv_off, w.n_kv_heads, w.page_size,
                                           1 / math.sqrt(d))
        o = out[n].float().cpu().numpy()
        live = np.ones(len(o), bool)
        live[q_off[4]:q_off[5]] = False    # empty context
        if dtype == "f32":
            assert np.abs(o[live] - ref[live]).max() <= 1e-5
        else:
            ok, st = bf16_close(o[live], ref[live])
            assert ok, st
        assert (o[~live] == 0).all()
        lg = lse[n].cpu().numpy()
        assert np.isneginf(lg[~live]).all()
        np.testing.assert_allclose(lg[live], rl[live], atol=1e-4)


@pytest.mark.parametrize("hkv", [2, 4], ids=["g4-packed", "g2-shared-kernel"])
@pytest.mark.parametrize("case", ["mixed", "no-affix", "all-private", "short", "many", "wide"])
def test_shared_affix_attention_seeded(case, hkv):
    """The shared-affix entry point on read tables that route a random part of
    the affix to the shared slots and the rest anywhere in the pool, with
    ragged queries (an empty request, a single row, B not a multiple of 4)
    and contexts (one shorter than the affix end, an empty one).  Its result
    is defined by the read table alone: same oracle as acache_mapped_attention.
    With 4 query heads per KV head a 32-row block fills a packed 128-row tile
    and the call runs the single pass; with 2 it runs the shared-affix kernel
    (four requests per workgroup: the "wide" case's 11 requests leave its
    third group one request short)."""
    nb = 11 if case == "wide" else 7
    w = Workload(101, "sh", "bf16", 2, 8, hkv, 128, (("req", 40), ("affix", 333), ("gen", 64)), nb, 0.2,
                 page_order="random")
    K = A.acache_anchor_count(w.L, w.rate)
    lay = gen.make_layout(w, K, 5)
    k, v = gen.make_pool(w, lay, device=DEV, seed=5)
    nslot = lay.n_pages * w.page_size
    rng = np.random.default_rng(17)
    l, L = w.affix_l, w.L
    shared = lay.shared_slots.astype(np.int32)
    T = [437, 437, 300, 437, 0, 437, 41]                 # request 2 ends inside the affix, 4 is empty
    q_counts = [32, 0, 17, 32, 5, 1, 32]
    if case == "many":
        q_counts = [32] * 7
    if case == "wide":
        T += [437, 200, 437, 437]
        q_counts += [32, 9, 0, 32]
    tables = []
    for b, t in enumerate(T):
        rs = rng.integers(0, nslot, t).astype(np.int32)
        if case != "all-private":
            j = np.arange(max(0, min(t - l, L)))
            keep = rng.random(len(j)) < (0.8 if case != "many" else 0.97)
            rs[l + j[keep]] = shared[j[keep]]
        tables.append(rs)
    read = np.concatenate(tables).astype(np.int32)
    kv_off = np.concatenate([[0], np.cumsum(T)]).astype(np.int32)
    q_off = np.concatenate([[0], np.cumsum(q_counts)]).astype(np.int32)
    qd = gen.make_rows(w, int(q_off[-1]), gen.S_QDEC, device=DEV, heads=w.n_q_heads, seed=5)
    ss = shared if case != "no-affix" else shared[:0]
    torch.cuda.synchronize()
    kh, vh, qh = np_of(k), np_of(v), np_of(qd)
    out = torch.full_like(qd, 7.0)
    lse = torch.empty(qd.shape[:3], device=DEV)
    A.acache_mapped_attention_shared(k, v, qd, i32(q_off), i32(read), i32(kv_off), i32(ss), out, lse=lse,
                                     affix_l=l, max_q_per_req=max(q_counts), max_kv_per_req=max(T))
    torch.cuda.synchronize()
    for n in range(w.n_layers):
        ref, rl = O.mapped_attention_layer(qh[n], kh[n], vh[n], q_off, read, kv_off, w.n_kv_heads, w.page_size,
                                           1 / math.sqrt(w.head_dim))
        o = out[n].float().cpu().numpy()
        live = np.ones(len(o), bool)
        live[q_off[4]:q_off[5]] = False    # empty context
        ok, st = bf16_close(o[live], ref[live])
        assert ok, st
        assert (o[~live] == 0).all()
        lg = lse[n].cpu().numpy()
        assert np.isneginf(lg[~live]).all()
        np.testing.assert_allclose(lg[live], rl[live], atol=1e-4)


@pytest.mark.parametrize("hq,hkv", [(28, 4), (8, 2), (8, 4), (32, 2), (16, 1)],
                         ids=["g7-packed", "g4-packed", "g2-unpacked", "g16-packed", "g16-mqa-packed"])
def test_gqa_decode_attention_packed(hq, hkv):
    """Decode blocks of grouped-query heads: with hq/hkv query heads per KV
    head and 32-row blocks, groups of 7 and 4 fill a 128-row tile and run
    packed (a unit's rows are (head, query) pairs of one KV-head group, the
    last tile partly empty); a group of 2 runs unpacked.  Ragged blocks (an
    empty one, a single row, rows not a multiple of 32) and contexts (one
    key, an empty context, one over several tiles with a ragged tail)."""
    w = Workload(103, "gq", "bf16", 2, hq, hkv, 128, (("req", 30), ("affix", 200), ("gen", 64)), 6, 0.2,
                 page_order="random")
    K = A.acache_anchor_count(w.L, w.rate)
    lay = gen.make_layout(w, K, 7)
    k, v = gen.make_pool(w, lay, device=DEV, seed=7)
    nslot = lay.n_pages * w.page_size
    rng = np.random.default_rng(23)
    q_counts = [32, 0, 17, 1, 32, 9]
    kv_counts = [294, 40, 1, 0, 130, 777]
    read = np.concatenate([rng.integers(0, nslot, c) for c in kv_counts]).astype(np.int32)
    q_off = np.concatenate([[0], np.cumsum(q_counts)]).astype(np.int32)
    kv_off = np.concatenate([[0], np.cumsum(kv_counts)]).astype(np.int32)
    qd = gen.make_rows(w, int(q_off[-1]), gen.S_QDEC, device=DEV, heads=w.n_q_heads, seed=7)
    torch.cuda.synchronize()
    kh, vh, qh = np_of(k), np_of(v), np_of(qd)
    out = torch.full_like(qd, 7.0)
    lse = torch.empty(qd.shape[:3], device=DEV)
    A.acache_mapped_attention(k, v, qd, i32(q_off), i32(read), i32(kv_off), out, lse=lse,
                              max_q_per_req=max(q_counts), max_kv_per_req=max(kv_counts))
    torch.cuda.synchronize()
    live = np.ones(int(q_off[-1]), bool)
    live[q_off[3]:q_off[4]] = False        # empty context
    for n in range(w.n_layers):
        ref, rl = O.mapped_attention_layer(qh[n], kh[n], vh[n], q_off, read, kv_off, w.n_kv_heads, w.page_size,
                                           1 / math.sqrt(w.head_dim))
        o = out[n].float().cpu().numpy()
        ok, st = bf16_close(o[live], ref[live])
        assert ok, (n, st)
        assert (o[~live] == 0).all()
        lg = lse[n].cpu().numpy()
        assert np.isneginf(lg[~live]).all()
        np.testing.assert_allclose(lg[live], rl[live], atol=1e-4)


@pytest.mark.parametrize("dtype,d,hq,hkv", [("bf16", 128, 4, 4), ("bf16", 128, 6, 2), ("bf16", 128, 8, 2),
                                             ("f32", 32, 4, 2)],
                         ids=["bf16-mha-one-kernel", "bf16-gqa3-two-calls", "bf16-gqa4-two-calls", "f32-two-calls"])
def test_store_attend_seeded(dtype, d, hq, hkv):
    """Store-then-attend of the recompute phase (Section 4.3): the pool after
    the call equals the oracle's scatter byte for byte, and the attention
    equals the oracle's read-slot attention over that pool.  Maps come from
    the oracle on seeded anchors.  Request 1 stores nothing (its recompute
    positions keep the pool's old rows), request 2 has no query rows (its rows
    must still be stored), request 0 has many query rows over several tiles."""
    _store_attend_case(dtype, d, hq, hkv, 0.2)


@pytest.mark.parametrize("rate", [0.0, 0.103, 0.105, 1.0],
                         ids=["no-anchors", "fresh-rows-end-on-a-tile", "one-fresh-row-past-a-tile",
                              "every-affix-position"])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 8)], ids=["mha4", "mha8"])
def test_store_attend_anchor_rates(hq, hkv, rate):
    """The same at the ratio extremes (Section 4.3 with ratio 0 and 1) and
    where the fresh rows meet the pool keys: with no anchors only the
    request's own positions are stored; at ratio 0.103 a storing request has
    128 fresh rows, two whole 64-key tiles, so no tile of the one-kernel path
    mixes fresh rows and pool slots; at 0.105 it has 129, one row into the
    next tile; with every affix position an anchor the storing requests read
    nothing but their fresh rows (an affix of 200, so that the 297 fresh
    rows take the 32-row kernel; test_store_attend_row_limit covers the
    48-row one)."""
    _store_attend_case("bf16", 128, hq, hkv, rate, affix=200 if rate == 1.0 else 300)


@pytest.mark.parametrize("anchors,affix", [(286, 400), (287, 400), (2975, 3000), (2976, 3000)],
                         ids=["383-rows-32-row-kernel", "384-rows-48-row-kernel", "3072-rows-48-row-kernel",
                              "3073-rows-two-calls"])
def test_store_attend_row_limit(anchors, affix):
    """The one kernel takes at most 3072 query rows per request
    (max_q_per_req): the 32-row tile loop below 384 rows, the 48-row kernel
    from 384; one row more than 3072 and the call makes the two calls of its
    definition.  Each side of both edges stores the rows byte for byte and
    attends as the oracle: request 0 recomputes 97 own positions plus its
    anchors, all of them query rows."""
    _store_attend_case("bf16", 128, 4, 4, anchors / affix, affix=affix, expect_rows=anchors + 97)


def _store_attend_case(dtype, d, hq, hkv, rate, affix=300, expect_rows=None):
    w = Workload(104, "sa", dtype, 2, hq, hkv, d, (("req", 24), ("affix", affix), ("req", 9), ("gen", 64)), 4, rate,
                 page_order="random")
    K = A.acache_anchor_count(w.L, w.rate)
    lay = gen.make_layout(w, K, 9)
    k, v = gen.make_pool(w, lay, device=DEV, seed=9)
    scores = gen.seeded_scores(w, seed=9).numpy().astype(np.float64)
    read, rc_pos, rc_slot, kept = [], [], [], [0]
    for b in range(w.batch):
        an = O.topk_anchors(scores[b], K, w.affix_l)
        pp = lay.private_pages[lay.private_page_offsets[b]:lay.private_page_offsets[b + 1]]
        r_, p_, s_ = O.build_maps(an, int(lay.seq_len[b]), w.affix_l, w.L, lay.shared_slots, pp, w.page_size)
        read.append(r_)
        if b != 1:
            rc_pos.append(p_)
            rc_slot.append(s_)
        kept.append(kept[-1] + (0 if b == 1 else len(p_)))
    read, rc_pos, rc_slot = (np.concatenate(x).astype(np.int32) for x in (read, rc_pos, rc_slot))
    src_off = np.array(kept, np.int32)
    n_src = int(src_off[-1])
    src_k = gen.make_rows(w, n_src, gen.S_SRC_K, device=DEV, seed=9)
    src_v = gen.make_rows(w, n_src, gen.S_SRC_V, device=DEV, seed=9)
    q_counts = [int(np.diff(lay.rc_offsets)[0]), 33, 0, 17]
    q_off = np.concatenate([[0], np.cumsum(q_counts)]).astype(np.int32)
    q = gen.make_rows(w, int(q_off[-1]), gen.S_QRC, device=DEV, heads=w.n_q_heads, seed=9)
    torch.cuda.synchronize()
    kh, vh, qh, skh, svh = np_of(k), np_of(v), np_of(q), np_of(src_k), np_of(src_v)
    if expect_rows is not None:
        assert max(q_counts) == expect_rows
        one_kernel = A.acache_store_attend_workspace_bytes(k, v, B=w.batch, max_q_per_req=max(q_counts),
                                                           max_kv_per_req=w.T) > 0
        assert one_kernel == (expect_rows <= 3072)
    out = torch.full_like(q, 7.0)
    lse = torch.empty(q.shape[:3], device=DEV)
    A.acache_store_attend(k, v, src_k, src_v, i32(rc_pos), i32(rc_slot), i32(src_off), q, i32(q_off), i32(read),
                          i32(lay.kv_offsets), out, lse=lse, max_q_per_req=max(q_counts), max_kv_per_req=w.T)
    torch.cuda.synchronize()
    kp, vp = kh.copy(), vh.copy()
    O.scatter(kp, vp, skh, svh, rc_slot, w.page_size)
    assert np.array_equal(np_of(k), kp) and np.array_equal(np_of(v), vp)
    for n in range(w.n_layers):
        ref, rl = O.mapped_attention_layer(qh[n], kp[n], vp[n], q_off, read, lay.kv_offsets, w.n_kv_heads,
                                           w.page_size, 1 / math.sqrt(d))
        o = out[n].float().cpu().numpy()
        if dtype == "f32":
            assert np.abs(o - ref).max() <= 1e-5
        else:
            ok, st = bf16_close(o, ref)
            assert ok, (n, st)
        np.testing.assert_allclose(lse[n].cpu().numpy(), rl, atol=1e-4)


def test_shared_affix_attention_matches_single_pass_and_repeats():
    """Two calls in a row (the second with fewer requests) agree with the
    single-pass entry point on a maps-built decode step."""
    w = Workload(102, "sh2", "bf16", 2, 8, 8, 128, (("affix", 512), ("req", 24), ("gen", 64)), 9, 0.2,
                 page_order="random", key_tweak="sinks")
    c = Chain(w, seed=3)
    c.run_gpu()
    for B in (w.batch, 5):
        q_off = i32(c.q_off[:B + 1])
        kv_off = i32(c.lay.kv_offsets[:B + 1])
        n_q = int(c.q_off[B])
        qd = c.qd[:, :n_q].contiguous()
        o1 = torch.empty_like(qd)
        o2 = torch.empty_like(qd)
        l1 = torch.empty(qd.shape[:3], device=DEV)
        l2 = torch.empty_like(l1)
        A.acache_mapped_attention(c.k, c.v, qd, q_off, c.read_slot, kv_off, o1, lse=l1, max_q_per_req=c.n_dec,
                                  max_kv_per_req=w.T)
        A.acache_mapped_attention_shared(c.k, c.v, qd, q_off, c.read_slot, kv_off, i32(c.lay.shared_slots), o2,
                                         lse=l2, affix_l=w.affix_l, max_q_per_req=c.n_dec, max_kv_per_req=w.T)
        torch.cuda.synchronize()
        # the two differ in summation order and in the running maxima the bf16
        # weights are taken against: held to the bar both meet against the oracle
        ok, st = bf16_close(o2.float().cpu().numpy(), o1.float().cpu().numpy())
        assert ok, (B, st)
        assert (l1 - l2).abs().max().item() <= 1e-4


def test_identity_map_matches_contiguous_sdpa_on_gpu():
    """Rate 0, prefix affix, natural page order: the library's read-slot map
    is the identity and its attention equals torch SDPA (fp64, CPU) over the
    contiguous pool."""
    w = Workload(99, "id", "bf16", 1, 4, 4, 128, (("affix", 96), ("req", 16), ("gen", 32)), 1, 0.0,
                 page_order="identity")
    c = Chain(w)
    c.run_gpu()
    assert c.read_slot.cpu().numpy().tolist() == list(range(w.T))
    c.run_oracle()   # the oracle's own scatter of the same sources gives the pool the attention reads
    kk = torch.from_numpy(c.r_kpool[0].view(np.int16)).view(torch.bfloat16).double()
    vv = torch.from_numpy(c.r_vpool[0].view(np.int16)).view(torch.bfloat16).double()
    kf = kk.permute(1, 0, 2, 3).reshape(w.n_kv_heads, -1, w.head_dim)[:, :w.T]
    vf = vv.permute(1, 0, 2, 3).reshape(w.n_kv_heads, -1, w.head_dim)[:, :w.T]
    qf = torch.from_numpy(c.h["qd"][0].view(np.int16)).view(torch.bfloat16).double().permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qf[None], kf[None], vf[None])[0].permute(1, 0, 2)
    ok, st = bf16_close(c.out[0].float().cpu().numpy(), ref.numpy())
    assert ok, st


def test_physical_permutation_bit_identical():
    """Permuting the physical slots (and remapping the table) gives the same
    output bits: the kernel walks keys in logical order."""
    w = Workload(100, "perm", "bf16", 1, 8, 8, 128, (("affix", 256), ("req", 32), ("gen", 32)), 2, 0.2,
                 page_order="random")
    K = A.acache_anchor_count(w.L, w.rate)
    lay = gen.make_layout(w, K, 8)
    k, v = gen.make_pool(w, lay, device=DEV)
    nslot = lay.n_pages * w.page_size
    rng = np.random.default_rng(12)
    read = np.concatenate([rng.permutation(nslot)[:w.T] for _ in range(w.batch)]).astype(np.int32)
    kv_off = (np.arange(w.batch + 1) * w.T).astype(np.int32)
    q_off = (np.arange(w.batch + 1) * 32).astype(np.int32)
    qd = gen.make_rows(w, 64, gen.S_QDEC, device=DEV, heads=w.n_q_heads)
    out1 = torch.empty_like(qd)
    A.acache_mapped_attention(k, v, qd, i32(q_off), i32(read), i32(kv_off), out1, max_q_per_req=32,
                              max_kv_per_req=w.T)
    perm = torch.as_tensor(rng.permutation(nslot), device=DEV)
    kf = k.permute(0, 1, 3, 2, 4).reshape(1, nslot, w.n_kv_heads, w.head_dim)
    vf = v.permute(0, 1, 3, 2, 4).reshape(1, nslot, w.n_kv_heads, w.head_dim)
    k2f = torch.empty_like(kf); v2f = torch.empty_like(vf)
    k2f[:, perm] = kf
    v2f[:, perm] = vf
    k2 = k2f.reshape(1, lay.n_pages, w.page_size, w.n_kv_heads, w.head_dim).permute(0, 1, 3, 2, 4).contiguous()
    v2 = v2f.reshape(1, lay.n_pages, w.page_size, w.n_kv_heads, w.head_dim).permute(0, 1, 3, 2, 4).contiguous()
    read2 = perm.cpu().numpy()[read].astype(np.int32)
    out2 = torch.empty_like(qd)
    A.acache_mapped_attention(k2, v2, qd, i32(q_off), i32(read2), i32(kv_off), out2, max_q_per_req=32,
                              max_kv_per_req=w.T)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def test_probe_is_deterministic_and_accumulates():
    """Two probe calls on the same inputs give identical bits, and a second
    call adds its layers' mass (Eq. 5 summed over layer groups)."""
    w = SMALL[1][1]
    c = Chain(w)
    lay = c.lay
    args = (c.k, c.v)
    s1 = torch.zeros((w.batch, w.L), device=DEV)
    s2 = torch.zeros((w.batch, w.L), device=DEV)
    for s in (s1, s2):
        A.acache_probe_scores(*args, c.q, i32(lay.masked_rows), i32(lay.masked_offsets), i32(lay.shared_slots), s,
                              max_masked=w.m)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    s3 = torch.zeros((w.batch, w.L), device=DEV)
    for n in range(w.n_layers):
        A.acache_probe_scores(*args, c.q[n:n + 1], i32(lay.masked_rows), i32(lay.masked_offsets),
                              i32(lay.shared_slots), s3, max_masked=w.m, layer_begin=n)
    torch.cuda.synchronize()
    np.testing.assert_allclose(s3.cpu().numpy(), s1.cpu().numpy(), rtol=1e-5)


@pytest.mark.parametrize("dtype,d,hq,hkv", [("bf16", 128, 4, 2), ("f32", 64, 3, 3)])
def test_column_mass_ragged_masked_sets(dtype, d, hq, hkv):
    """Eq. (4)-(5) with ragged masked sets per request: none, one row, exactly
    one 32-row tile, a ragged tail over several tiles, a request with none
    between two that have rows.  scores accumulate (+=): a request without
    masked rows keeps its initial value.  A second call in which no request
    has a masked row leaves scores unchanged."""
    w = Workload(121, "ragged-mask", dtype, 2, hq, hkv, d, (("affix", 300), ("req", 20), ("gen", 70)), 7, 0.2,
                 page_order="random")
    K = A.acache_anchor_count(w.L, w.rate)
    lay = gen.make_layout(w, K, 4)
    k, v = gen.make_pool(w, lay, device=DEV, seed=4)
    q = gen.make_probe_q(w, lay, device=DEV, seed=4)
    counts = [0, 1, 32, 0, 70, 45, 0]
    rng = np.random.default_rng(4)
    rows, off = [], [0]
    for b, c in enumerate(counts):
        r0, r1 = int(lay.row_offsets[b]), int(lay.row_offsets[b + 1])
        rows += sorted(rng.choice(np.arange(r0, r1), size=c, replace=False).tolist())
        off.append(len(rows))
    rows, off = np.array(rows, np.int32), np.array(off, np.int32)
    scores = torch.full((w.batch, w.L), 0.5, device=DEV)
    A.acache_probe_scores(k, v, q, i32(rows), i32(off), i32(lay.shared_slots), scores, max_masked=max(counts))
    torch.cuda.synchronize()
    got = scores.cpu().numpy().astype(np.float64)
    kh, vh, qh = np_of(k), np_of(v), np_of(q)
    ref = np.full((w.batch, w.L), 0.5)
    for n in range(w.n_layers):
        ref += O.probe_layer(qh[n], kh[n], vh[n], lay.shared_slots, w.page_size, w.n_kv_heads, rows, off,
                             1 / math.sqrt(d), want_out=False)[2]
    for b, c in enumerate(counts):
        if c == 0:
            assert (got[b] == 0.5).all(), f"request {b} has no masked rows"
    rel = np.abs(got - ref) / ref
    assert rel.max() <= (1e-5 if dtype == "f32" else 1e-3), rel.max()
    np.testing.assert_allclose(got.sum(axis=1), 0.5 * w.L + w.n_layers * hq * np.array(counts), rtol=1e-4)
    # no masked rows anywhere: nothing is added
    before = scores.clone()
    A.acache_probe_scores(k, v, q, torch.empty(0, dtype=torch.int32, device=DEV),
                          torch.zeros(w.batch + 1, dtype=torch.int32, device=DEV), i32(lay.shared_slots), scores,
                          max_masked=0)
    torch.cuda.synchronize()
    assert torch.equal(scores, before)


def test_calls_on_other_streams():
    """Every call takes the stream to run on (a torch stream or a raw
    handle); workspaces the binding allocates itself live on that stream.
    An admission and a decode step (probe, Top-K and maps, store-then-attend,
    shared-affix read-slot attention) on a side stream equal the same calls
    on the current stream, bit for bit."""
    w = SMALL[1][1]
    c = Chain(w, seed=5)
    lay = c.lay
    max_r = int(np.diff(lay.rc_offsets).max())
    keep = [i32(x) for x in (lay.seq_len, lay.shared_slots, lay.private_pages, lay.private_page_offsets,
                             lay.kv_offsets, lay.rc_offsets, lay.masked_rows, lay.masked_offsets)]
    qr = gen.make_rows(w, c.n_rc, gen.S_QRC, device=DEV, heads=w.n_q_heads, seed=5)

    def run(stream):
        k, v = c.k.clone(), c.v.clone()
        scores = torch.zeros((w.batch, w.L), device=DEV)
        anchors = torch.empty((w.batch, c.K), dtype=torch.int32, device=DEV)
        read = torch.empty(int(lay.kv_offsets[-1]), dtype=torch.int32, device=DEV)
        rcp = torch.empty(c.n_rc, dtype=torch.int32, device=DEV)
        rcs = torch.empty_like(rcp)
        orc = torch.empty_like(qr)
        out = torch.empty_like(c.qd)
        maps = A.map_args(w.batch, w.affix_l, w.L, c.K, w.page_size, w.T, *keep[:6], read, rcp, rcs)
        torch.cuda.synchronize()   # the copies and fills above are done before another stream reads them
        A.acache_probe_scores(k, v, c.q, keep[6], keep[7], keep[1], scores, max_masked=w.m, stream=stream)
        A.acache_topk_anchors(scores, c.K, w.affix_l, anchors, maps, stream=stream)
        A.acache_store_attend(k, v, c.src_k, c.src_v, rcp, rcs, keep[5], qr, keep[5], read, keep[4], orc,
                              max_q_per_req=max_r, max_kv_per_req=w.T, stream=stream)
        A.acache_mapped_attention_shared(k, v, c.qd, i32(c.q_off), read, keep[4], keep[1], out, affix_l=w.affix_l,
                                         max_q_per_req=c.n_dec, max_kv_per_req=w.T, stream=stream)
        return scores, anchors, orc, out, k, v

    ref = run(None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for stream in (side, side.cuda_stream):
        got = run(stream)
        torch.cuda.synchronize()
        for name, x, y in zip(("scores", "anchors", "store-then-attend O", "shared-affix O", "pool k", "pool v"),
                              got, ref):
            assert torch.equal(x, y), f"{name} on stream {stream!r}"


@pytest.mark.parametrize("scale", [0.03, 0.7])
def test_softmax_scale_is_honoured(scale):
    """Every call takes the softmax scale (Eq. 4 divides by sqrt(d) by
    default); a scale far below and far above it gives the oracle's probe
    scores, O_aff and LSE, and the oracle's read-slot attention through both
    read-slot calls."""
    w = SMALL[1][1]
    c = Chain(w, seed=6)
    lay, h = c.lay, c.h
    scores = torch.zeros((w.batch, w.L), device=DEV)
    o_aff = torch.empty_like(c.q)
    lse_aff = torch.empty(c.q.shape[:3], device=DEV)
    A.acache_probe_scores(c.k, c.v, c.q, i32(lay.masked_rows), i32(lay.masked_offsets), i32(lay.shared_slots),
                          scores, max_masked=w.m, o_aff=o_aff, lse_aff=lse_aff, scale=scale)
    read = np.concatenate([O.build_maps(np.arange(c.K) + w.affix_l, int(lay.seq_len[b]), w.affix_l, w.L,
                                        lay.shared_slots,
                                        lay.private_pages[lay.private_page_offsets[b]:lay.private_page_offsets[b + 1]],
                                        w.page_size)[0] for b in range(w.batch)])
    out = torch.empty_like(c.qd)
    lse = torch.empty(c.qd.shape[:3], device=DEV)
    out_sh = torch.empty_like(c.qd)
    lse_sh = torch.empty(c.qd.shape[:3], device=DEV)
    A.acache_mapped_attention(c.k, c.v, c.qd, i32(c.q_off), i32(read), i32(lay.kv_offsets), out, lse=lse,
                              max_q_per_req=c.n_dec, max_kv_per_req=w.T, scale=scale)
    A.acache_mapped_attention_shared(c.k, c.v, c.qd, i32(c.q_off), i32(read), i32(lay.kv_offsets),
                                     i32(lay.shared_slots), out_sh, lse=lse_sh, affix_l=w.affix_l,
                                     max_q_per_req=c.n_dec, max_kv_per_req=w.T, scale=scale)
    torch.cuda.synchronize()
    s_ref = np.zeros((w.batch, w.L))
    for n in range(w.n_layers):
        o_r, l_r, s_n = O.probe_layer(h["q"][n], h["k"][n], h["v"][n], lay.shared_slots, w.page_size, w.n_kv_heads,
                                      lay.masked_rows, lay.masked_offsets, scale)
        s_ref += s_n
        ok, st = bf16_close(o_aff[n].float().cpu().numpy(), o_r)
        assert ok, f"O_aff layer {n}: {st}"
        np.testing.assert_allclose(lse_aff[n].cpu().numpy(), l_r, atol=1e-4)
        o_m, l_m = O.mapped_attention_layer(h["qd"][n], h["k"][n], h["v"][n], c.q_off, read, lay.kv_offsets,
                                            w.n_kv_heads, w.page_size, scale)
        for name, got_o, got_l in (("single pass", out, lse), ("shared affix", out_sh, lse_sh)):
            ok, st = bf16_close(got_o[n].float().cpu().numpy(), o_m)
            assert ok, f"{name} O layer {n}: {st}"
            np.testing.assert_allclose(got_l[n].cpu().numpy(), l_m, atol=1e-4)
    s_gpu = scores.cpu().numpy().astype(np.float64)
    big = s_ref >= 1e-6 * s_ref.max()
    assert (np.abs(s_gpu - s_ref)[big] / s_ref[big]).max() <= 1e-3


def test_layer_subset_calls_match_whole_calls():
    """A call over layers layer_begin .. layer_begin+n-1 (q holding only those
    layers) computes what the whole-stack call computes for them, bit for
    bit: the probe, both read-slot calls and the column mass."""
    w = SMALL[2][1]
    c = Chain(w, seed=8)
    c.run_gpu()
    lay = c.lay
    for n in range(w.n_layers):
        q1, qd1 = c.q[n:n + 1].contiguous(), c.qd[n:n + 1].contiguous()
        o_aff = torch.empty_like(q1)
        lse_aff = torch.empty(q1.shape[:3], device=DEV)
        A.acache_probe_attention(c.k, c.v, q1, i32(lay.shared_slots), lse_aff, o_aff=o_aff, layer_begin=n)
        out = torch.empty_like(qd1)
        out_sh = torch.empty_like(qd1)
        A.acache_mapped_attention(c.k, c.v, qd1, i32(c.q_off), c.read_slot, i32(lay.kv_offsets), out,
                                  max_q_per_req=c.n_dec, max_kv_per_req=w.T, layer_begin=n)
        A.acache_mapped_attention_shared(c.k, c.v, qd1, i32(c.q_off), c.read_slot, i32(lay.kv_offsets),
                                         i32(lay.shared_slots), out_sh, affix_l=w.affix_l, max_q_per_req=c.n_dec,
                                         max_kv_per_req=w.T, layer_begin=n)
        torch.cuda.synchronize()
        assert torch.equal(o_aff[0], c.o_aff[n]), f"probe O_aff, layer {n}"
        assert torch.equal(lse_aff[0], c.lse_aff[n]), f"probe LSE, layer {n}"
        assert torch.equal(out[0], c.out[n]), f"single-pass read-slot attention, layer {n}"
        assert torch.equal(out_sh[0], c.out_sh[n]), f"shared-affix read-slot attention, layer {n}"


@pytest.mark.parametrize("idx", [1, 2])
def test_dropna_attention(idx):
    """DropNA (Section 5.3): the recompute map doubles as the read table with
    the non-anchor affix cache dropped.  The library's recompute slots equal
    the oracle's DropNA tables bit for bit, and the read-slot attention over
    them matches the oracle's attention over those tables."""
    name, w = SMALL[idx]
    c = Chain(w, n_dec=min(w.block_len, w.m), seed=7)
    c.run_gpu()
    c.run_oracle()
    an = c.anchors.cpu().numpy()
    for b in range(w.batch):
        assert anchors_match(c.r_scores[b], an[b], c.K, w.affix_l)[0]
    if any(an[b].tolist() != c.r_anchors[b].tolist() for b in range(w.batch)):
        # the sets differ only inside the tie band: the oracle's tables follow the library's anchors
        c.run_oracle_downstream(list(an), c.r_layers)
    lay = c.lay
    dn = [O.dropna_read_table(c.r_read[lay.kv_offsets[b]:lay.kv_offsets[b + 1]], c.r_anchors_used[b], w.affix_l,
                              w.L) for b in range(w.batch)]
    assert np.array_equal(c.rc_slot.cpu().numpy(), np.concatenate(dn))
    out = torch.empty_like(c.qd)
    lse = torch.empty(c.qd.shape[:3], device=DEV)
    A.acache_mapped_attention(c.k, c.v, c.qd, i32(c.q_off), c.rc_slot, i32(lay.rc_offsets), out, lse=lse,
                              max_q_per_req=c.n_dec, max_kv_per_req=int(np.diff(lay.rc_offsets).max()))
    torch.cuda.synchronize()
    dn_off = np.concatenate([[0], np.cumsum([len(x) for x in dn])])
    for i, n in enumerate(c.r_layers):
        ref, rl = O.mapped_attention_layer(c.h["qd"][n], c.r_kpool[i], c.r_vpool[i], c.q_off, np.concatenate(dn),
                                           dn_off, w.n_kv_heads, w.page_size, c.scale)
        ok, st = bf16_close(out[n].float().cpu().numpy(), ref)
        assert ok, f"DropNA attention layer {n}: {st}"
        np.testing.assert_allclose(lse[n].cpu().numpy(), rl, atol=1e-4)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 32)])
def test_lse_merge_seeded(dtype, d):
    """The merge of two attentions over disjoint key sets against the
    oracle's definition, with empty parts (-inf) and in-place outputs."""
    g = torch.Generator().manual_seed(11)
    n, H = 37, 6
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    oa = torch.randn(n, H, d, generator=g).to(dt).to(DEV)
    ob = torch.randn(n, H, d, generator=g).to(dt).to(DEV)
    la = (torch.randn(n, H, generator=g) * 3).to(DEV)
    lb = (torch.randn(n, H, generator=g) * 3).to(DEV)
    la[0, :] = -math.inf
    lb[1, :] = -math.inf
    la[2, :] = -math.inf
    lb[2, :] = -math.inf
    h = [np_of(x) for x in (oa, la, ob, lb)]
    o = torch.empty_like(oa)
    l = torch.empty_like(la)
    A.acache_lse_merge(la, lb, l, oa, ob, o)
    ref_o, ref_l = O.lse_merge(O.decode(h[0]) if dtype == "bf16" else h[0].astype(np.float64), h[1].astype(np.float64),
                               O.decode(h[2]) if dtype == "bf16" else h[2].astype(np.float64), h[3].astype(np.float64))
    torch.cuda.synchronize()
    got = o.float().cpu().numpy()
    if dtype == "bf16":
        ok, st = bf16_close(got, ref_o)
        assert ok, st
    else:
        assert np.abs(got - ref_o).max() <= 1e-5
    np.testing.assert_allclose(l.cpu().numpy(), ref_l, atol=1e-5)
    assert (got[2] == 0).all() and np.isneginf(l[2].cpu().numpy()).all()
    A.acache_lse_merge(la, lb, la, oa, ob, oa)      # in place
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16 if dtype == "bf16" else torch.int32),
                       o.view(torch.int16 if dtype == "bf16" else torch.int32))
    assert torch.equal(la, l)


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_probe_full_normaliser_chain(idx):
    """The full-context reading of the probe normaliser through the library:
    probe attention over the affix, read-slot attention of the same rows over
    their own non-affix keys, LSE merge, column mass with the merged LSE.
    O, LSE and scores against the oracle's one-softmax formulation, and the
    anchor sets under this reading against the oracle's.  Then the same
    normaliser in one pass (each request's rows over its affix slots followed
    by its own slots) against the same oracle values."""
    name, w = SMALL[idx]
    K = A.acache_anchor_count(w.L, w.rate)
    lay = gen.make_layout(w, K, 9)
    k, v = gen.make_pool(w, lay, device=DEV, seed=9)
    q = gen.make_probe_q(w, lay, device=DEV, seed=9)
    na, na_off = [], [0]
    for b in range(w.batch):
        pp = lay.private_pages[lay.private_page_offsets[b]:lay.private_page_offsets[b + 1]]
        P_b = int(lay.row_offsets[b + 1] - lay.row_offsets[b])
        na += [int(pp[i // w.page_size]) * w.page_size + i % w.page_size for i in range(P_b)]
        na_off.append(len(na))
    na, na_off = np.array(na, np.int32), np.array(na_off, np.int32)
    torch.cuda.synchronize()
    hk, hv, hq = np_of(k), np_of(v), np_of(q)
    scale = 1 / math.sqrt(w.head_dim)
    o_aff = torch.empty_like(q)
    lse_aff = torch.empty(q.shape[:3], device=DEV)
    A.acache_probe_attention(k, v, q, i32(lay.shared_slots), lse_aff, o_aff=o_aff)
    o_na = torch.empty_like(q)
    lse_na = torch.empty_like(lse_aff)
    max_p = int(np.diff(lay.row_offsets).max())
    A.acache_mapped_attention(k, v, q, i32(lay.row_offsets), i32(na), i32(na_off), o_na, lse=lse_na,
                              max_q_per_req=max_p, max_kv_per_req=max_p)
    A.acache_lse_merge(lse_aff, lse_na, lse_aff, o_aff, o_na, o_aff)
    scores = torch.zeros((w.batch, w.L), device=DEV)
    A.acache_probe_column_mass(k, v, q, i32(lay.masked_rows), i32(lay.masked_offsets), i32(lay.shared_slots),
                               lse_aff, scores, max_masked=w.m)
    torch.cuda.synchronize()
    fp32 = w.dtype == "f32"
    s_ref = np.zeros((w.batch, w.L))
    refs = {}
    for n in range(w.n_layers):
        of, lf, sf = O.probe_layer_full(hq[n], hk[n], hv[n], lay.shared_slots, lay.row_offsets, na, na_off,
                                        w.page_size, w.n_kv_heads, lay.masked_rows, lay.masked_offsets, scale)
        refs[n] = (of, lf)
        s_ref += sf
        got = np_of(o_aff[n]).astype(np.float64) if fp32 else o_aff[n].float().cpu().numpy()
        if fp32:
            assert np.abs(got - of).max() <= 1e-5
        else:
            # three bf16 roundings stand between this output and the exact one (P inside each part,
            # each part's O as stored, the merged O), one more than a single attention: up to
            # 3 * 2^-9 * max|V|, which exceeds 2e-2 where an output nears the largest |V| (measured
            # 0.0216 on this case); the one-pass formulation below holds the 2e-2 bar
            vmax = float(np.abs(O.decode(hv[n])).max())
            ok, st = bf16_close(got, of, max_abs=3 * 2.0 ** -9 * vmax)
            assert ok, f"full-normaliser O layer {n}: {st}"
        np.testing.assert_allclose(lse_aff[n].cpu().numpy(), lf, atol=1e-4)
    s_gpu = scores.cpu().numpy().astype(np.float64)
    big = s_ref >= 1e-6 * s_ref.max()
    assert (np.abs(s_gpu - s_ref)[big] / s_ref[big]).max() <= (1e-5 if fp32 else 1e-3)
    assert (s_gpu.sum(axis=1) < w.n_layers * w.n_q_heads * np.diff(lay.masked_offsets)).all()
    an = torch.empty((w.batch, K), dtype=torch.int32, device=DEV)
    A.acache_topk_anchors(scores, K, w.affix_l, an)
    torch.cuda.synchronize()
    for b in range(w.batch):
        ok, _ = anchors_match(s_ref[b], an.cpu().numpy()[b], K, w.affix_l)
        assert ok
    # the same normaliser in one pass: each request's rows attend to the
    # affix slots followed by their own slots (one softmax, no merge)
    one, one_off = [], [0]
    for b in range(w.batch):
        one += list(lay.shared_slots) + list(na[na_off[b]:na_off[b + 1]])
        one_off.append(len(one))
    o1 = torch.empty_like(q)
    l1 = torch.empty_like(lse_aff)
    A.acache_mapped_attention(k, v, q, i32(lay.row_offsets), i32(np.array(one, np.int32)),
                              i32(np.array(one_off, np.int32)), o1, lse=l1, max_q_per_req=max_p,
                              max_kv_per_req=w.L + max_p)
    s1 = torch.zeros((w.batch, w.L), device=DEV)
    A.acache_probe_column_mass(k, v, q, i32(lay.masked_rows), i32(lay.masked_offsets), i32(lay.shared_slots),
                               l1, s1, max_masked=w.m)
    torch.cuda.synchronize()
    for n in range(w.n_layers):
        of, lf = refs[n]
        got = np_of(o1[n]).astype(np.float64) if fp32 else o1[n].float().cpu().numpy()
        if fp32:
            assert np.abs(got - of).max() <= 1e-5
        else:
            ok, st = bf16_close(got, of)
            assert ok, f"one-pass full-normaliser O layer {n}: {st}"
        np.testing.assert_allclose(l1[n].cpu().numpy(), lf, atol=1e-4)
    s1 = s1.cpu().numpy().astype(np.float64)
    assert (np.abs(s1 - s_ref)[big] / s_ref[big]).max() <= (1e-5 if fp32 else 1e-3)


@pytest.mark.parametrize("wl", ["small-f32", "small-bf16", "dream-gqa-L2048"])
def test_hkvd_scores_and_anchors(wl):
    """HKVD deviation scores (Appendix B.5) against the oracle, and the anchor
    sets their Top-K selects."""
    if wl == "small-f32":
        w = SMALL[3][1]
    elif wl == "small-bf16":
        w = SMALL[1][1]
    else:
        w = WORKLOADS[3]
    K = A.acache_anchor_count(w.L, w.rate)
    lay = gen.make_layout(w, K, 4)
    k, v = gen.make_pool(w, lay, device=DEV, seed=4)
    dt = gen.TORCH_DT[w.dtype]
    g = torch.Generator(device=DEV).manual_seed(21)
    shape = (w.n_layers, w.batch, w.L, w.n_kv_heads, w.head_dim)
    kf = torch.randn(shape, generator=g, device=DEV).to(dt)
    vf = torch.randn(shape, generator=g, device=DEV).to(dt)
    scores = torch.zeros((w.batch, w.L), device=DEV)
    A.acache_hkvd_scores(k, v, i32(lay.shared_slots), kf, vf, scores)
    torch.cuda.synchronize()
    ref = O.hkvd_scores(np_of(k), np_of(v), lay.shared_slots, np_of(kf), np_of(vf), w.page_size)
    got = scores.cpu().numpy().astype(np.float64)
    assert (np.abs(got - ref) / ref).max() <= 1e-5
    an = torch.empty((w.batch, K), dtype=torch.int32, device=DEV)
    A.acache_topk_anchors(scores, K, w.affix_l, an)
    torch.cuda.synchronize()
    for b in range(w.batch):
        ok, _ = anchors_match(ref[b], an.cpu().numpy()[b], K, w.affix_l)
        assert ok
