"""The path inside a HIP graph: one decode step (probe, Top-K and maps,
admission scatter, block store, shared-affix read-slot attention), and one
admission (probe, Top-K and maps, store-then-attend), each captured once and
replayed.  The library enqueues kernels only (no memset, copy,
allocation or synchronisation), so a serving loop can capture it; every
replay must reproduce the eager step bit for bit (all of its kernels are
deterministic).  Eager work and synchronisations run between the replays."""
import numpy as np
import pytest
import torch

import attention_anchor_probe_amd as A
from synth.configs import Workload
from synth import gen
from tests.gpu_common import DEV, i32

pytestmark = pytest.mark.gpu


def test_decode_step_in_a_hip_graph():
    w = Workload(105, "graph", "bf16", 2, 4, 4, 128, (("affix", 256), ("req", 24), ("gen", 64)), 5, 0.2,
                 page_order="random")
    K = A.acache_anchor_count(w.L, w.rate)
    lay = gen.make_layout(w, K, 11)
    k, v = gen.make_pool(w, lay, device=DEV, seed=11)
    q = gen.make_probe_q(w, lay, device=DEV, seed=11)
    n_rc = int(lay.rc_offsets[-1])
    src_k = gen.make_rows(w, n_rc, gen.S_SRC_K, device=DEV, seed=11)
    src_v = gen.make_rows(w, n_rc, gen.S_SRC_V, device=DEV, seed=11)
    nb = w.batch * w.block_len
    qd = gen.make_rows(w, nb, gen.S_QDEC, device=DEV, heads=w.n_q_heads, seed=11)
    bk = gen.make_rows(w, nb, gen.S_BLK_K, device=DEV, seed=11)
    bv = gen.make_rows(w, nb, gen.S_BLK_V, device=DEV, seed=11)
    tabs = [i32(x) for x in (lay.seq_len, lay.shared_slots, lay.private_pages, lay.private_page_offsets,
                             lay.kv_offsets, lay.rc_offsets, lay.masked_rows, lay.masked_offsets)]
    q_off = i32(np.arange(w.batch + 1) * w.block_len)
    bstart = i32(np.full(w.batch, gen.block_positions(w, 0)[0], np.int32))
    # outputs and workspaces, allocated before the capture
    scores = torch.empty((w.batch, w.L), device=DEV)
    o_aff = torch.empty_like(q)
    lse_aff = torch.empty(q.shape[:3], device=DEV)
    anchors = torch.empty((w.batch, K), dtype=torch.int32, device=DEV)
    read_slot = torch.empty(int(lay.kv_offsets[-1]), dtype=torch.int32, device=DEV)
    rc_pos = torch.empty(n_rc, dtype=torch.int32, device=DEV)
    rc_slot = torch.empty_like(rc_pos)
    dst = torch.empty(nb, dtype=torch.int32, device=DEV)
    out = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], device=DEV)
    ws_probe = torch.empty(A.acache_probe_workspace_bytes(q.shape[1], w.batch, w.L, w.n_q_heads, w.n_layers, True),
                           dtype=torch.uint8, device=DEV)
    ws_map = torch.empty(max(1, A.acache_mapped_attention_shared_workspace_bytes(
        k, v, B=w.batch, n_q=nb, max_q_per_req=w.block_len, n_q_heads=w.n_q_heads, n_layers=w.n_layers,
        max_kv_per_req=w.T, L=w.L)), dtype=torch.uint8, device=DEV)
    maps = A.map_args(w.batch, w.affix_l, w.L, K, w.page_size, w.T, *tabs[:6], read_slot, rc_pos, rc_slot)
    outputs = (scores, o_aff, lse_aff, anchors, read_slot, rc_pos, rc_slot, dst, out, lse, k, v)

    def step():
        scores.zero_()
        A.acache_probe_scores(k, v, q, tabs[6], tabs[7], tabs[1], scores, max_masked=w.m, o_aff=o_aff,
                              lse_aff=lse_aff, workspace=ws_probe)
        A.acache_topk_anchors(scores, K, w.affix_l, anchors, maps)
        A.acache_scatter_private(k, v, src_k, src_v, rc_slot)
        A.acache_block_slots(read_slot, tabs[4], bstart, w.block_len, dst)
        A.acache_scatter_private(k, v, bk, bv, dst)
        A.acache_mapped_attention_shared(k, v, qd, q_off, read_slot, tabs[4], tabs[1], out, lse=lse,
                                         affix_l=w.affix_l, max_q_per_req=w.block_len, max_kv_per_req=w.T,
                                         workspace=ws_map)

    # eager step: the reference bits
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]

    # capture (after a warm-up on the capture's side stream, as torch advises)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for replay in range(3):
        # eager work between the replays, and the outputs cleared so that a
        # replay that wrote nothing would be caught
        for t in (scores, o_aff, lse_aff, out, lse):
            t.fill_(-7.0)
        for t in (anchors, read_slot, rc_pos, rc_slot, dst):
            t.fill_(-1)
        x = torch.randn(512, 512, device=DEV)
        (x @ x).sum().item()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("scores", "o_aff", "lse_aff", "anchors", "read_slot", "rc_pos", "rc_slot", "dst",
                                    "out", "lse", "pool k", "pool v"), outputs, ref):
            assert torch.equal(got, want), f"replay {replay}: {name} differs from the eager step"


def test_admission_in_a_hip_graph():
    """The admission path captured once: probe, Top-K and maps, then the
    recompute phase's store-then-attend in one call (the recomputed rows
    stored to their private slots while the recompute queries attend through
    the read-slot map).  The call writes only slots it does not read, so a
    replay over its own output pool is idempotent; every replay reproduces the
    eager admission bit for bit."""
    w = Workload(106, "graph-admission", "bf16", 2, 4, 2, 128, (("req", 16), ("affix", 256), ("gen", 48)), 3, 0.2,
                 page_order="random")
    K = A.acache_anchor_count(w.L, w.rate)
    lay = gen.make_layout(w, K, 12)
    k, v = gen.make_pool(w, lay, device=DEV, seed=12)
    q = gen.make_probe_q(w, lay, device=DEV, seed=12)
    n_rc = int(lay.rc_offsets[-1])
    src_k = gen.make_rows(w, n_rc, gen.S_SRC_K, device=DEV, seed=12)
    src_v = gen.make_rows(w, n_rc, gen.S_SRC_V, device=DEV, seed=12)
    qr = gen.make_rows(w, n_rc, gen.S_QRC, device=DEV, heads=w.n_q_heads, seed=12)
    tabs = [i32(x) for x in (lay.seq_len, lay.shared_slots, lay.private_pages, lay.private_page_offsets,
                             lay.kv_offsets, lay.rc_offsets, lay.masked_rows, lay.masked_offsets)]
    max_r = int(np.diff(lay.rc_offsets).max())
    scores = torch.empty((w.batch, w.L), device=DEV)
    anchors = torch.empty((w.batch, K), dtype=torch.int32, device=DEV)
    read_slot = torch.empty(int(lay.kv_offsets[-1]), dtype=torch.int32, device=DEV)
    rc_pos = torch.empty(n_rc, dtype=torch.int32, device=DEV)
    rc_slot = torch.empty_like(rc_pos)
    out = torch.empty_like(qr)
    lse = torch.empty(qr.shape[:3], device=DEV)
    ws_probe = torch.empty(A.acache_probe_workspace_bytes(q.shape[1], w.batch, w.L, w.n_q_heads, w.n_layers, False),
                           dtype=torch.uint8, device=DEV)
    ws_store = torch.empty(max(1, A.acache_store_attend_workspace_bytes(k, v, B=w.batch, max_q_per_req=max_r,
                                                                        max_kv_per_req=w.T)),
                           dtype=torch.uint8, device=DEV)
    maps = A.map_args(w.batch, w.affix_l, w.L, K, w.page_size, w.T, *tabs[:6], read_slot, rc_pos, rc_slot)
    outputs = (scores, anchors, read_slot, rc_pos, rc_slot, out, lse, k, v)

    def admission():
        scores.zero_()
        A.acache_probe_scores(k, v, q, tabs[6], tabs[7], tabs[1], scores, max_masked=w.m, workspace=ws_probe)
        A.acache_topk_anchors(scores, K, w.affix_l, anchors, maps)
        A.acache_store_attend(k, v, src_k, src_v, rc_pos, rc_slot, tabs[5], qr, tabs[5], read_slot, tabs[4], out,
                              lse=lse, max_q_per_req=max_r, max_kv_per_req=w.T, workspace=ws_store)

    admission()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        admission()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        admission()
    torch.cuda.synchronize()

    for replay in range(3):
        for t in (scores, out, lse):
            t.fill_(-7.0)
        for t in (anchors, read_slot, rc_pos, rc_slot):
            t.fill_(-1)
        x = torch.randn(512, 512, device=DEV)
        (x @ x).sum().item()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("scores", "anchors", "read_slot", "rc_pos", "rc_slot", "out", "lse", "pool k",
                                    "pool v"), outputs, ref):
            assert torch.equal(got, want), f"replay {replay}: {name} differs from the eager admission"
