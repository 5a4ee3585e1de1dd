"""Helpers of the GPU parity tests: run the library's chain and the oracle's
own chain on the same seeded inputs and compare stage by stage.

The oracle receives generator inputs (copied to the host before the library
touches them).  One library output is fed back, in compositional checks
only: where the library's anchor set differs from the oracle's inside the
tie band (after both have been compared against the oracle's scores), the
oracle's maps, scatter and attention are recomputed from the library's
anchors, so that those stages are still checked on that seed.
"""
import math

import numpy as np
import torch

import attention_anchor_probe_amd as A
from oracle import acache_oracle as O
from synth import gen
from tests.helpers import np_of

DEV = "cuda:0"


def i32(a):
    return gen.to_device_i32(a, DEV)


def anchors_match(s_ref, an_gpu, K, affix_l, rel_band=1e-3):
    """Anchor-set agreement.  Exact when the oracle's K-th gap exceeds
    rel_band relative; otherwise offsets whose oracle score lies outside
    s_K * (1 +- rel_band) must be classified identically.  Returns (ok, exact)."""
    s_ref = np.asarray(s_ref, np.float64)
    L = len(s_ref)
    got = set(int(a) - affix_l for a in an_gpu)
    if len(got) != K or any(j < 0 or j >= L for j in got):
        return False, False
    want = set(int(a) - affix_l for a in O.topk_anchors(s_ref, K, affix_l))
    if got == want:
        return True, True
    if K == 0 or K == L:
        return False, False
    srt = np.sort(s_ref)[::-1]
    sK, sK1 = srt[K - 1], srt[K]
    if sK > 0 and (sK - sK1) / sK > rel_band:
        return False, False
    lo, hi = sK * (1 - rel_band), sK * (1 + rel_band)
    for j in range(L):
        if s_ref[j] > hi and j not in got:
            return False, False
        if s_ref[j] < lo and j in got:
            return False, False
    return True, False


def bf16_close(out, ref, max_abs=2e-2, mean_abs=1e-3, rms_rel=1e-2):
    out = np.asarray(out, np.float64)
    err = np.abs(out - ref)
    rms_ref = math.sqrt(float((ref ** 2).mean())) if ref.size else 0.0
    rms_err = math.sqrt(float((err ** 2).mean())) if err.size else 0.0
    ok = err.max(initial=0) <= max_abs and err.mean() <= mean_abs if err.size else True
    ok = ok and (rms_err <= rms_rel * rms_ref + 1e-30)
    return ok, dict(max_abs=float(err.max(initial=0)), mean_abs=float(err.mean()) if err.size else 0.0,
                    rms_err=rms_err, rms_ref=rms_ref)


class Chain:
    """One seeded workload instance: inputs on the GPU, host snapshots for
    the oracle, and the library's outputs."""

    def __init__(self, w, seed=0, page_order=None, shared_slot_order=None, n_dec=None):
        self.w = w
        self.K = A.acache_anchor_count(w.L, w.rate)
        assert self.K == O.anchor_count(w.L, w.rate)
        self.lay = gen.make_layout(w, self.K, seed, page_order=page_order, shared_slot_order=shared_slot_order)
        lay = self.lay
        self.k, self.v = gen.make_pool(w, lay, device=DEV, seed=seed)
        self.q = gen.make_probe_q(w, lay, device=DEV, seed=seed)
        self.n_rc = int(lay.rc_offsets[-1])
        self.src_k = gen.make_rows(w, self.n_rc, gen.S_SRC_K, device=DEV, seed=seed)
        self.src_v = gen.make_rows(w, self.n_rc, gen.S_SRC_V, device=DEV, seed=seed)
        self.n_dec = w.block_len if n_dec is None else n_dec
        self.qd = gen.make_rows(w, w.batch * self.n_dec, gen.S_QDEC, device=DEV, seed=seed, heads=w.n_q_heads)
        self.q_off = np.arange(w.batch + 1) * self.n_dec
        torch.cuda.synchronize()
        self.h = {name: np_of(getattr(self, name)) for name in ("k", "v", "q", "src_k", "src_v", "qd")}
        self.scale = 1.0 / math.sqrt(w.head_dim)

    # ---------------------------------------------------------------- library
    def run_gpu(self):
        w, lay, K = self.w, self.lay, self.K
        self.scores = torch.zeros((w.batch, w.L), device=DEV)
        self.o_aff = torch.empty_like(self.q)
        self.lse_aff = torch.empty(self.q.shape[:3], device=DEV)
        A.acache_probe_scores(self.k, self.v, self.q, i32(lay.masked_rows), i32(lay.masked_offsets),
                              i32(lay.shared_slots), self.scores, max_masked=w.m, o_aff=self.o_aff,
                              lse_aff=self.lse_aff)
        self.anchors = torch.empty((w.batch, K), dtype=torch.int32, device=DEV)
        self.read_slot = torch.empty(int(lay.kv_offsets[-1]), dtype=torch.int32, device=DEV)
        self.rc_pos = torch.empty(self.n_rc, dtype=torch.int32, device=DEV)
        self.rc_slot = torch.empty_like(self.rc_pos)
        self._keep = [i32(x) for x in (lay.seq_len, lay.shared_slots, lay.private_pages, lay.private_page_offsets,
                                       lay.kv_offsets, lay.rc_offsets)]
        maps = A.map_args(w.batch, w.affix_l, w.L, K, w.page_size, w.T, *self._keep, self.read_slot, self.rc_pos,
                          self.rc_slot)
        A.acache_topk_anchors(self.scores, K, w.affix_l, self.anchors, maps)
        A.acache_scatter_private(self.k, self.v, self.src_k, self.src_v, self.rc_slot)
        self.out = torch.empty_like(self.qd)
        self.lse = torch.empty(self.qd.shape[:3], device=DEV)
        A.acache_mapped_attention(self.k, self.v, self.qd, i32(self.q_off), self.read_slot, i32(lay.kv_offsets),
                                  self.out, lse=self.lse, max_q_per_req=self.n_dec, max_kv_per_req=w.T)
        # the same attention through the shared-affix entry point
        self.out_sh = torch.empty_like(self.qd)
        self.lse_sh = torch.empty(self.qd.shape[:3], device=DEV)
        A.acache_mapped_attention_shared(self.k, self.v, self.qd, i32(self.q_off), self.read_slot,
                                         i32(lay.kv_offsets), self._keep[1], self.out_sh, lse=self.lse_sh,
                                         affix_l=w.affix_l, max_q_per_req=self.n_dec, max_kv_per_req=w.T)
        torch.cuda.synchronize()

    # ----------------------------------------------------------------- oracle
    def run_oracle(self, layers=None):
        w, lay, K, h = self.w, self.lay, self.K, self.h
        layers = list(range(w.n_layers)) if layers is None else layers
        self.r_scores = np.zeros((w.batch, w.L))
        self.r_oaff, self.r_lseaff = {}, {}
        for n in range(w.n_layers):
            o, lse, s = O.probe_layer(h["q"][n], h["k"][n], h["v"][n], lay.shared_slots, w.page_size, w.n_kv_heads,
                                      lay.masked_rows, lay.masked_offsets, self.scale, want_out=n in layers)
            self.r_scores += s
            if n in layers:
                self.r_oaff[n], self.r_lseaff[n] = o, lse
        self.r_anchors = [O.topk_anchors(self.r_scores[b], K, w.affix_l) for b in range(w.batch)]
        self.run_oracle_downstream(self.r_anchors, layers)

    def run_oracle_downstream(self, anchors, layers=None):
        """The oracle's maps, scatter and read-slot attention from the anchor
        sets `anchors` (the oracle's own, or the library's once they have been
        checked against the oracle's scores up to the tie band)."""
        w, lay, h = self.w, self.lay, self.h
        layers = list(range(w.n_layers)) if layers is None else layers
        self.r_anchors_used = [np.asarray(a) for a in anchors]
        rd, rp, rs = [], [], []
        for b in range(w.batch):
            pp = lay.private_pages[lay.private_page_offsets[b]:lay.private_page_offsets[b + 1]]
            r_, p_, s_ = O.build_maps(self.r_anchors_used[b], int(lay.seq_len[b]), w.affix_l, w.L,
                                      lay.shared_slots, pp, w.page_size)
            rd.append(r_); rp.append(p_); rs.append(s_)
        self.r_read, self.r_rcpos, self.r_rcslot = map(np.concatenate, (rd, rp, rs))
        kp, vp = h["k"][layers].copy(), h["v"][layers].copy()
        O.scatter(kp, vp, h["src_k"][layers], h["src_v"][layers], self.r_rcslot, w.page_size)
        self.r_kpool, self.r_vpool, self.r_layers = kp, vp, layers
        self.r_out, self.r_lse = {}, {}
        for i, n in enumerate(layers):
            self.r_out[n], self.r_lse[n] = O.mapped_attention_layer(
                h["qd"][n], kp[i], vp[i], self.q_off, self.r_read, lay.kv_offsets, w.n_kv_heads, w.page_size,
                self.scale)
