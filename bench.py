"""Benchmark of the ACache slot-mapped attention path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input
shaped like LLaDA-8B attention with a shared prefix affix of L=4096 tokens
(32 layers, 32 heads, head_dim 128, 16 requests, 256 request tokens and 256
generation tokens each, anchor ratio 0.2 -> K=820):

  1. probe attention     O_aff, LSE_aff of the 16*512 non-affix rows over the affix
  2. probe column mass   Eq. (4) weights of the 16*256 masked rows summed into scores
  3. Top-K + maps        anchors (Eq. 6), read-slot and recompute maps
  4. admission scatter   recomputed K/V of anchors + request positions -> private slots
  5. block store         the 32-row decode block's K/V -> its private slots
  6. read-slot attention 16 x 32 block queries over T=4608 logical keys (the
     shared-affix call: the affix is read once per group of four requests)

Inputs are generated on the GPU from fixed seeds and are resident in HBM when
the timed region starts.  Prints one JSON line.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import attention_anchor_probe_amd as A  # noqa: E402
from synth.configs import WORKLOADS, BENCH_WORKLOAD  # noqa: E402
from synth import gen  # noqa: E402

METRIC = "mapped-attention TFLOP/s (% bf16 MFMA peak); probe ms/request at affix L=4096"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=BENCH_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--steps-only", action="store_true",
                    help="skip the measurements after the timed steps (single-pass, recompute, DropNA, "
                         "full-normaliser and HKVD timings), so that a profile holds the steps' launches only")
    ap.add_argument("--ceilings", action="store_true",
                    help="also time a large library bf16 GEMM and torch's fused attention at the probe's per-layer "
                         "shape on the same GPU: context for the probe kernel's MFMA rate, not part of the path")
    ap.add_argument("--shared-slot-order", choices=("page", "slot"), default=None,
                    help="order of the shared region's slots: whole pages (the workloads' default) or a slot-granular "
                         "shuffle, the worst case for the read-slot attention's gathers")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device copy of this many MiB before the steps (counter calibration)")
    return ap.parse_args()


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Setup:
    def __init__(self, w, dev):
        self.w, self.dev = w, dev
        self.K = A.acache_anchor_count(w.L, w.rate)
        lay = self.lay = gen.make_layout(w, self.K, seed=0)
        i32 = lambda a: gen.to_device_i32(a, dev)
        self.k, self.v = gen.make_pool(w, lay, device=dev)
        self.q = gen.make_probe_q(w, lay, device=dev)
        self.n_rows = self.q.shape[1]
        self.n_rc = int(lay.rc_offsets[-1])
        self.src_k = gen.make_rows(w, self.n_rc, gen.S_SRC_K, device=dev)
        self.src_v = gen.make_rows(w, self.n_rc, gen.S_SRC_V, device=dev)
        nb = w.batch * w.block_len
        self.qd = gen.make_rows(w, nb, gen.S_QDEC, device=dev, heads=w.n_q_heads)
        self.blk_k = gen.make_rows(w, nb, gen.S_BLK_K, device=dev)
        self.blk_v = gen.make_rows(w, nb, gen.S_BLK_V, device=dev)
        self.masked_rows, self.masked_offsets = i32(lay.masked_rows), i32(lay.masked_offsets)
        self.shared_slots = i32(lay.shared_slots)
        self.kv_offsets = i32(lay.kv_offsets)
        self.q_off = i32(np.arange(w.batch + 1) * w.block_len)
        self.block_start = i32(np.full(w.batch, gen.block_positions(w, 0)[0], np.int32))
        # outputs and workspaces
        self.o_aff = torch.empty_like(self.q)
        self.lse_aff = torch.empty(self.q.shape[:3], device=dev)
        self.scores = torch.zeros((w.batch, w.L), device=dev)
        ws = A.acache_probe_column_mass_workspace_bytes(self.q.shape[1], w.batch, w.L, w.n_q_heads, w.n_layers)
        self.ws = torch.empty(ws, dtype=torch.uint8, device=dev)
        self.anchors = torch.empty((w.batch, self.K), dtype=torch.int32, device=dev)
        self.read_slot = torch.empty(int(lay.kv_offsets[-1]), dtype=torch.int32, device=dev)
        self.rc_pos = torch.empty(self.n_rc, dtype=torch.int32, device=dev)
        self.rc_slot = torch.empty_like(self.rc_pos)
        self._keep = [i32(x) for x in (lay.seq_len, lay.shared_slots, lay.private_pages, lay.private_page_offsets,
                                       lay.kv_offsets, lay.rc_offsets)]
        self.maps = A.map_args(w.batch, w.affix_l, w.L, self.K, w.page_size, w.T, *self._keep, self.read_slot,
                               self.rc_pos, self.rc_slot)
        self.blk_dst = torch.empty(nb, dtype=torch.int32, device=dev)
        self.out = torch.empty_like(self.qd)
        ws = A.acache_mapped_attention_shared_workspace_bytes(
            self.k, self.v, B=w.batch, n_q=nb, max_q_per_req=w.block_len, n_q_heads=w.n_q_heads,
            n_layers=w.n_layers, max_kv_per_req=w.T, L=w.L)
        self.ws_map = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    STAGES = ("probe_attention", "probe_column_mass", "topk_maps", "admission_scatter", "block_store",
              "mapped_attention")

    def step(self, ev):
        """One pass of the path; ev[i] is recorded after stage i (ev[0] before)."""
        w = self.w
        ev[0].record()
        A.acache_probe_attention(self.k, self.v, self.q, self.shared_slots, self.lse_aff, o_aff=self.o_aff)
        ev[1].record()
        self.scores.zero_()
        A.acache_probe_column_mass(self.k, self.v, self.q, self.masked_rows, self.masked_offsets, self.shared_slots,
                                   self.lse_aff, self.scores, max_masked=w.m, workspace=self.ws)
        ev[2].record()
        A.acache_topk_anchors(self.scores, self.K, w.affix_l, self.anchors, self.maps)
        ev[3].record()
        A.acache_scatter_private(self.k, self.v, self.src_k, self.src_v, self.rc_slot)
        ev[4].record()
        A.acache_block_slots(self.read_slot, self.kv_offsets, self.block_start, w.block_len, self.blk_dst)
        A.acache_scatter_private(self.k, self.v, self.blk_k, self.blk_v, self.blk_dst)
        ev[5].record()
        A.acache_mapped_attention_shared(self.k, self.v, self.qd, self.q_off, self.read_slot, self.kv_offsets,
                                         self.shared_slots, self.out, affix_l=w.affix_l, max_q_per_req=w.block_len,
                                         max_kv_per_req=w.T, workspace=self.ws_map)
        ev[6].record()

    def extra_layers(self):
        """Layers the recompute-phase timings run on: all of them when their
        queries and outputs fit in half of the free device memory beside the
        step's buffers, else the first that do (the L=16384 workload)."""
        w = self.w
        per_layer = 2 * self.n_rc * w.n_q_heads * w.head_dim * (2 if w.dtype == "bf16" else 4)
        free, _ = torch.cuda.mem_get_info()
        return max(1, min(w.n_layers, int(0.5 * free) // per_layer))

    def recompute_ms(self, reps, nl):
        """Recompute-phase read-slot attention (Section 4.3): queries only for
        every request's recomputed rows (anchors and request positions),
        keys and values through the read-slot map; layers 0 .. nl-1, timed on
        its own."""
        w = self.w
        qr = gen.make_rows(w, self.n_rc, gen.S_QRC, device=self.dev, heads=w.n_q_heads, layers=range(nl))
        orc = torch.empty_like(qr)
        max_r = int(np.diff(self.lay.rc_offsets).max())
        rc_off = self._keep[5]
        run = lambda: A.acache_mapped_attention(self.k, self.v, qr, rc_off, self.read_slot, self.kv_offsets, orc,
                                                max_q_per_req=max_r, max_kv_per_req=w.T)
        run()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            run()
            ev[i + 1].record()
        torch.cuda.synchronize()
        del qr, orc
        return float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))

    def store_attend_ms(self, reps, nl):
        """The admission's store-then-attend in one call (Section 4.3): the
        recomputed K/V rows of every request are stored to their private slots
        and the recompute-phase queries attend through the read-slot map,
        reading those rows from the source; layers 0 .. nl-1, timed on its
        own."""
        w = self.w
        qr = gen.make_rows(w, self.n_rc, gen.S_QRC, device=self.dev, heads=w.n_q_heads, layers=range(nl))
        orc = torch.empty_like(qr)
        max_r = int(np.diff(self.lay.rc_offsets).max())
        rc_off = self._keep[5]
        nb = A.acache_store_attend_workspace_bytes(self.k, self.v, B=w.batch, max_q_per_req=max_r,
                                                   max_kv_per_req=w.T)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=self.dev)
        run = lambda: A.acache_store_attend(self.k, self.v, self.src_k[:nl], self.src_v[:nl], self.rc_pos,
                                            self.rc_slot, rc_off, qr, rc_off, self.read_slot, self.kv_offsets, orc,
                                            max_q_per_req=max_r, max_kv_per_req=w.T, workspace=ws)
        run()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            run()
            ev[i + 1].record()
        torch.cuda.synchronize()
        del qr, orc, ws
        return float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))

    def dropna_ms(self, reps):
        """Decode-block attention under the DropNA ablation (Section 5.3): the
        same queries over the recompute map only (the non-anchor affix cache
        dropped); timed on its own."""
        w = self.w
        max_r = int(np.diff(self.lay.rc_offsets).max())
        run = lambda: A.acache_mapped_attention(self.k, self.v, self.qd, self.q_off, self.rc_slot, self._keep[5],
                                                self.out, max_q_per_req=w.block_len, max_kv_per_req=max_r)
        run()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            run()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))

    def full_normaliser(self):
        """The full-context reading of the probe normaliser: the non-affix rows'
        attention over their own non-affix keys (held here in the first P_b
        slots of each request's private pages), merged by LSE with the
        attention over the affix; the column mass and Top-K then run on the
        merged LSE.  Returns the extra time of the own-key attention and the
        merge, the mean overlap (|A n A'| / K) of the two anchor sets, and the
        time of the same probe attention done in one pass over each request's
        affix and own keys."""
        w, lay = self.w, self.lay
        na, na_off = [], [0]
        for b in range(w.batch):
            pp = lay.private_pages[lay.private_page_offsets[b]:lay.private_page_offsets[b + 1]]
            P_b = int(lay.row_offsets[b + 1] - lay.row_offsets[b])
            na += [int(pp[i // w.page_size]) * w.page_size + i % w.page_size for i in range(P_b)]
            na_off.append(len(na))
        i32 = lambda a: gen.to_device_i32(a, self.dev)
        na_off_h = np.array(na_off)
        na, na_off, row_off = i32(na), i32(na_off), i32(lay.row_offsets)
        max_p = int(np.diff(lay.row_offsets).max())
        o_na = torch.empty_like(self.q)
        lse_na = torch.empty_like(self.lse_aff)
        A.acache_probe_attention(self.k, self.v, self.q, self.shared_slots, self.lse_aff, o_aff=self.o_aff)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        A.acache_mapped_attention(self.k, self.v, self.q, row_off, na, na_off, o_na, lse=lse_na,
                                  max_q_per_req=max_p, max_kv_per_req=max_p)
        A.acache_lse_merge(self.lse_aff, lse_na, self.lse_aff, self.o_aff, o_na, self.o_aff)
        ev[1].record()
        scores = torch.zeros_like(self.scores)
        A.acache_probe_column_mass(self.k, self.v, self.q, self.masked_rows, self.masked_offsets, self.shared_slots,
                                   self.lse_aff, scores, max_masked=w.m, workspace=self.ws)
        an_full = torch.empty_like(self.anchors)
        A.acache_topk_anchors(scores, self.K, w.affix_l, an_full)
        torch.cuda.synchronize()
        a1, a2 = self.anchors.cpu().numpy(), an_full.cpu().numpy()
        overlap = float(np.mean([len(set(a1[b]) & set(a2[b])) / max(self.K, 1) for b in range(w.batch)]))
        del o_na, lse_na
        # the same normaliser in one pass: every request's rows over its affix
        # slots followed by its own slots (one softmax, no merge)
        na_h = na.cpu().numpy()
        one = np.concatenate([np.concatenate([lay.shared_slots, na_h[na_off_h[b]:na_off_h[b + 1]]])
                              for b in range(w.batch)])
        one_off = np.concatenate([[0], np.cumsum([w.L + na_off_h[b + 1] - na_off_h[b] for b in range(w.batch)])])
        one, one_off = i32(one), i32(one_off)
        o1 = torch.empty_like(self.q)
        l1 = torch.empty_like(self.lse_aff)
        run = lambda: A.acache_mapped_attention(self.k, self.v, self.q, row_off, one, one_off, o1, lse=l1,
                                                max_q_per_req=max_p, max_kv_per_req=w.L + max_p)
        run()
        ev2 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev2[0].record()
        run()
        ev2[1].record()
        torch.cuda.synchronize()
        del o1, l1
        return ev[0].elapsed_time(ev[1]), overlap, ev2[0].elapsed_time(ev2[1])

    def hkvd_ms(self, reps):
        """The CacheBlend-style HKVD selector scores (Appendix B.5) of every
        request's affix tokens over all layers, on synthetic full-prompt K/V
        of the same shape; timed on its own.  The full-prompt K/V of the first
        nb requests that fit in half of the free device memory are timed (all
        of them unless the workload is the L=16384 one) and the time scaled to
        every request.  Returns (ms, algorithmic GB, nb, the rate of the timed
        calls over the bytes they read: nb requests' K/V and the affix once)."""
        w = self.w
        per_req = 2 * w.n_layers * w.L * w.n_kv_heads * w.head_dim * 2
        free, _ = torch.cuda.mem_get_info()
        nb = max(1, min(w.batch, int(0.5 * free) // per_req))
        g = torch.Generator(device=self.dev).manual_seed(5)
        shape = (w.n_layers, nb, w.L, w.n_kv_heads, w.head_dim)
        kf = torch.randn(shape, generator=g, device=self.dev, dtype=torch.bfloat16)
        vf = torch.randn(shape, generator=g, device=self.dev, dtype=torch.bfloat16)
        sc = torch.zeros((nb, w.L), device=self.dev)
        A.acache_hkvd_scores(self.k, self.v, self.shared_slots, kf, vf, sc)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            A.acache_hkvd_scores(self.k, self.v, self.shared_slots, kf, vf, sc)
            ev[i + 1].record()
        torch.cuda.synchronize()
        # every request's full-prompt K/V once, and the shared affix K/V once
        affix = 2 * w.L * w.n_layers * w.n_kv_heads * w.head_dim * 2
        gb = (per_req * w.batch + affix) / 1e9
        del kf, vf, sc
        t = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))
        # a call on nb < B requests reads the affix once for nb requests, so
        # the scaled time charges it B / nb times; the timed calls' own rate:
        timed_gbs = (per_req * nb + affix) / 1e9 / (t * 1e-3)
        return t * w.batch / nb, gb, nb, timed_gbs

    def probe_single_request(self, reps):
        """The probe of one request alone at the same shapes (its non-affix
        rows over the affix in all layers, the column mass of its masked rows,
        its Top-K): the cost a request pays when no other request shares the
        affix.  Returns the mean ms of each part."""
        w, lay = self.w, self.lay
        r0, r1 = int(lay.row_offsets[0]), int(lay.row_offsets[1])
        m0, m1 = int(lay.masked_offsets[0]), int(lay.masked_offsets[1])
        i32 = lambda a: gen.to_device_i32(np.asarray(a, np.int32), self.dev)
        q1 = self.q[:, r0:r1].contiguous()
        o1 = torch.empty_like(q1)
        lse1 = torch.empty(q1.shape[:3], device=self.dev)
        mrows, moff = i32(lay.masked_rows[m0:m1] - r0), i32([0, m1 - m0])
        sc = torch.zeros((1, w.L), device=self.dev)
        ws = torch.empty(A.acache_probe_column_mass_workspace_bytes(q1.shape[1], 1, w.L, w.n_q_heads, w.n_layers),
                         dtype=torch.uint8, device=self.dev)
        an = torch.empty((1, self.K), dtype=torch.int32, device=self.dev)

        def run(ev):
            ev[0].record()
            A.acache_probe_attention(self.k, self.v, q1, self.shared_slots, lse1, o_aff=o1)
            ev[1].record()
            sc.zero_()
            A.acache_probe_column_mass(self.k, self.v, q1, mrows, moff, self.shared_slots, lse1, sc,
                                       max_masked=m1 - m0, workspace=ws)
            ev[2].record()
            A.acache_topk_anchors(sc, self.K, w.affix_l, an)
            ev[3].record()
        run([torch.cuda.Event(enable_timing=True) for _ in range(4)])
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
        for ev in evs:
            run(ev)
        torch.cuda.synchronize()
        part = lambda j: float(np.mean([ev[j].elapsed_time(ev[j + 1]) for ev in evs]))
        res = {"attention_ms": part(0), "column_mass_ms": part(1), "topk_ms": part(2)}
        res["ms"] = sum(res.values())
        del q1, o1, lse1, ws
        return res

    def mapped_cold_warm(self, reps, flush_mib=512):
        """The shared-affix read-slot attention timed warm (calls back to back)
        and cold (a flush_mib MiB buffer written between calls, so that no
        K/V row is left in L2 or the memory-side cache); median ms of each."""
        w = self.w
        run = lambda: A.acache_mapped_attention_shared(
            self.k, self.v, self.qd, self.q_off, self.read_slot, self.kv_offsets, self.shared_slots, self.out,
            affix_l=w.affix_l, max_q_per_req=w.block_len, max_kv_per_req=w.T, workspace=self.ws_map)
        flush = torch.empty(flush_mib << 20, dtype=torch.uint8, device=self.dev)
        res = {}
        for mode in ("warm", "cold"):
            ts = []
            for _ in range(reps):
                if mode == "cold":
                    flush.fill_(1)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                run()
                b.record()
                ts.append((a, b))
            torch.cuda.synchronize()
            res[f"{mode}_ms"] = float(np.median([a.elapsed_time(b) for a, b in ts]))
        del flush
        return res

    def single_pass_ms(self, reps):
        """The same read-slot attention through the single-pass entry point
        (every request streams its whole read list), timed on its own."""
        w = self.w
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            A.acache_mapped_attention(self.k, self.v, self.qd, self.q_off, self.read_slot, self.kv_offsets,
                                      self.out, max_q_per_req=w.block_len, max_kv_per_req=w.T)
            ev[i + 1].record()
        torch.cuda.synchronize()
        return float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))


def work_model(w, K):
    """Algorithmic FLOPs and bytes of each stage (what the method must compute
    or move; unique bytes of the workload's storage type)."""
    P, L, T, d, N, Hq, Hkv, B, m = w.P, w.L, w.T, w.head_dim, w.n_layers, w.n_q_heads, w.n_kv_heads, w.batch, w.m
    e = 2 if w.dtype == "bf16" else 4
    kv_bytes_per_pos = N * Hkv * d * e * 2          # K and V, all layers and KV heads
    rows = B * P
    q_bytes = N * rows * Hq * d * e
    probe_flops = 4.0 * rows * L * d * N * Hq        # QK^T and PV over the affix (O(N H P L))
    probe_bytes = L * kv_bytes_per_pos + 2 * q_bytes + N * rows * Hq * 4
    cm_flops = 2.0 * B * m * L * d * N * Hq          # recomputed q.k of the masked rows (O(N H m L))
    R = K + P
    scatter_bytes = 2 * B * R * kv_bytes_per_pos     # read sources, write slots
    nb = B * w.block_len
    mapped_flops = 4.0 * nb * T * d * N * Hq
    recompute_flops = 4.0 * B * R * T * d * N * Hq
    mapped_bytes = L * kv_bytes_per_pos + B * R * kv_bytes_per_pos + 2 * N * nb * Hq * d * e
    return dict(probe_flops=probe_flops, probe_bytes=probe_bytes, cm_flops=cm_flops, scatter_bytes=scatter_bytes,
                mapped_flops=mapped_flops, mapped_bytes=mapped_bytes, recompute_flops=recompute_flops,
                block_bytes=2 * nb * kv_bytes_per_pos)


TRAFFIC_SOURCES = ("k_attn_mfma.hip", "k_tables.hip")   # the sources of the counted kernels


def many_query_kernel(n_q_heads, n_kv_heads, max_q):
    """The kernel a bf16, head_dim 128 read-slot or probe attention launch
    takes, by the library's rule: the query heads of a KV-head group are
    packed into a unit's rows when the group has several and the requests
    have more than 32 rows or the group's rows reach 128; unpacked blocks of
    at most 32 rows take the single pass; units of at least 384 rows take the
    48-row kernel."""
    G = n_q_heads // n_kv_heads
    packed = G > 1 and (max_q > 32 or G * max_q >= 128)
    if not packed and max_q <= 32:
        return "attn_split_mfma"
    return "attn_rows48_mfma" if (G * max_q if packed else max_q) >= 384 else "attn_rows_mfma"


def code_digest(path):
    """sha256 of a kernel source without its comments and white space: it
    changes when the code changes, not when a comment does."""
    import hashlib
    import re
    txt = open(path).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    txt = re.sub(r"//[^\n]*", "", txt)
    return hashlib.sha256(re.sub(r"\s+", "", txt).encode()).hexdigest()


def measured_traffic(workload_name):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    runs (scaled by the counters' reading of a 1 GiB device copy), or {} (no
    figure) when the code of a counted kernel changed since the counters were
    taken."""
    path = os.path.join(ROOT, "profiles", f"pmc_traffic_{workload_name}.json")
    if not os.path.exists(path):
        return {}
    rec = json.load(open(path))
    digests = rec.get("code_sha256", {})
    for f in TRAFFIC_SOURCES:
        if code_digest(os.path.join(ROOT, "attention_anchor_probe_amd", "csrc", f)) != digests.get(f):
            return {}
    return {k: v["hbm_bytes"] for k, v in rec["kernels"].items()}


def cpu_baseline(w, S, host, target_s=10.0):
    """The fp64 oracle, as it stands, timed on the host's cores on a bounded
    sample of the same workload, grown layer by layer until each part has run
    for about target_s seconds: read-slot attention of all requests' decode
    blocks (maps built by the oracle from a seeded Top-K), and the probe of all
    requests' rows (extrapolated to all layers for ms/request)."""
    from oracle import acache_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    lay, K = S.lay, S.K
    scale = 1 / math.sqrt(w.head_dim)
    scores = gen.seeded_scores(w).numpy().astype(np.float64)
    anchors = [O.topk_anchors(scores[b], K, w.affix_l) for b in range(w.batch)]
    read = []
    for b in range(w.batch):
        pp = lay.private_pages[lay.private_page_offsets[b]:lay.private_page_offsets[b + 1]]
        read.append(O.build_maps(anchors[b], w.T, w.affix_l, w.L, lay.shared_slots, pp, w.page_size)[0])
    read = np.concatenate(read)
    q_off = np.arange(w.batch + 1) * w.block_len
    t_map, n_map = 0.0, 0
    for n in range(len(host["k"])):
        t0 = time.perf_counter()
        O.mapped_attention_layer(host["qd"][n], host["k"][n], host["v"][n], q_off, read, lay.kv_offsets,
                                 w.n_kv_heads, w.page_size, scale)
        t_map += time.perf_counter() - t0
        n_map += 1
        if t_map >= target_s:
            break
    mapped_flops = 4.0 * w.batch * w.block_len * w.T * w.head_dim * w.n_q_heads * n_map
    t_probe, n_probe = 0.0, 0
    for n in range(len(host["k"])):
        t0 = time.perf_counter()
        O.probe_layer(host["q"][n], host["k"][n], host["v"][n], lay.shared_slots, w.page_size, w.n_kv_heads,
                      lay.masked_rows, lay.masked_offsets, scale)
        t_probe += time.perf_counter() - t0
        n_probe += 1
        if t_probe >= target_s:
            break
    probe_ms_req = t_probe / n_probe * w.n_layers / w.batch * 1e3
    return {"value": mapped_flops / t_map / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": (f"read-slot attention of all {w.batch} requests x {w.block_len} queries x {w.n_q_heads} heads "
                       f"over T={w.T} keys on {n_map} of {w.n_layers} layers ({t_map:.1f} s); probe of all "
                       f"{w.batch * w.P} rows on {n_probe} of {w.n_layers} layers ({t_probe:.1f} s), its ms/request "
                       f"extrapolated to {w.n_layers} layers"),
            "probe_ms_per_request_extrapolated": probe_ms_req,
            "seconds": t_map + t_probe}


def library_ceilings(w, dev, reps=10):
    """What the installed libraries reach on this GPU for the same kind of
    work: a plain 4 GiB device copy (GB/s of bytes read plus written), a
    16384^3 bf16 GEMM (hipBLASLt through torch.matmul) and torch's
    fused attention kernels (flash and memory-efficient backends only, never
    the unfused math path) over one layer of the probe: all requests' non-affix
    rows of one request's shape against the affix, every head."""
    import torch.nn.functional as F
    from torch.nn.attention import sdpa_kernel, SDPBackend

    def t(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps
    res = {}
    # a plain 4 GiB device copy (read + write bytes): the practical HBM rate
    src = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    res["device_copy_gbs"] = 2.0 * src.numel() / t(lambda: dst.copy_(src)) / 1e6
    del src, dst
    n = 16384
    x = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    y = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    res["gemm_16384_bf16_tflops"] = 2.0 * n ** 3 / t(lambda: x @ y) / 1e9
    del x, y
    q = torch.randn(w.batch, w.n_q_heads, w.P, w.head_dim, device=dev, dtype=torch.bfloat16)
    k = torch.randn(w.batch, w.n_q_heads, w.L, w.head_dim, device=dev, dtype=torch.bfloat16)
    v = torch.randn_like(k)
    flop = 4.0 * w.batch * w.n_q_heads * w.P * w.L * w.head_dim
    for name, be in (("flash", SDPBackend.FLASH_ATTENTION), ("efficient", SDPBackend.EFFICIENT_ATTENTION)):
        try:
            with sdpa_kernel([be]):
                ms = t(lambda: F.scaled_dot_product_attention(q, k, v))
            res[f"sdpa_{name}_tflops"] = flop / ms / 1e9
        except RuntimeError as e:
            res[f"sdpa_{name}_unavailable"] = str(e)[:120]
    del q, k, v
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the path shards by request with no exchange, and this build "
              "runs and reports a single GPU only (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"
    w = WORKLOADS[args.workload]
    if args.shared_slot_order and args.shared_slot_order != w.shared_slot_order:
        w = w.scaled(shared_slot_order=args.shared_slot_order, name=f"{w.name}-{args.shared_slot_order}-granular")
    S = Setup(w, dev)
    progress(f"inputs of {w.name} resident")
    host = None
    if not args.no_cpu_baseline:
        def np_of(t):
            t = t.detach().cpu().contiguous()
            return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()
        n_snap = min(w.n_layers, 8)
        host = {"k": [np_of(S.k[n]) for n in range(n_snap)], "v": [np_of(S.v[n]) for n in range(n_snap)],
                "q": [np_of(S.q[n]) for n in range(n_snap)], "qd": [np_of(S.qd[n]) for n in range(n_snap)]}
    if args.calib_copy_mib:
        x = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
        del x, y
    nst = len(Setup.STAGES)
    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)]
    for _ in range(args.warmup):
        S.step(mk())
    torch.cuda.synchronize()
    progress(f"{args.warmup} warm-up steps done")
    evs = [mk() for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        S.step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    progress(f"{args.steps} timed steps done ({total_ms / args.steps:.2f} ms/step)")
    extras = {}
    stage_mean = lambda name: float(np.mean([evs[i][Setup.STAGES.index(name)].elapsed_time(
        evs[i][Setup.STAGES.index(name) + 1]) for i in range(args.steps)]))
    if not args.steps_only:
        single_ms = S.single_pass_ms(max(3, args.steps // 2))
        nl = S.extra_layers()
        rc_ms = S.recompute_ms(3, nl)
        sa_ms = S.store_attend_ms(3, nl)
        lf = w.n_layers / nl   # the recompute timings scale to all layers
        dropna_ms = S.dropna_ms(max(3, args.steps // 2))
        progress("single-pass, recompute, store-then-attend and DropNA timings done")
        fn_ms, fn_overlap, fn_one_ms = S.full_normaliser()
        hk_ms, hk_gb, hk_nb, hk_timed_gbs = S.hkvd_ms(3)
        progress("full-context normaliser and HKVD timings done")
        single_req = S.probe_single_request(max(3, args.steps // 2))
        cold_warm = S.mapped_cold_warm(max(5, args.steps))
        progress("single-request probe and cold/warm timings done")
        extras = {
            "probe_single_request": single_req,
            "mapped_attention_cold_warm": cold_warm,
            "mapped_attention_single_pass_ms": single_ms,
            "recompute_layers_timed": nl,
            "recompute_attention_ms": rc_ms * lf,
            "recompute_attention_tflops": work_model(w, S.K)["recompute_flops"] / lf / (rc_ms * 1e-3) / 1e12,
            "store_then_attend": {"one_call_ms": sa_ms * lf,
                                  "scatter_then_attention_ms": stage_mean("admission_scatter") + rc_ms * lf,
                                  "tflops": work_model(w, S.K)["recompute_flops"] / lf / (sa_ms * 1e-3) / 1e12},
            "dropna_mapped_attention_ms": dropna_ms,
            "full_normaliser": {"extra_ms": fn_ms, "anchor_overlap_with_affix_only": fn_overlap,
                                "one_pass_ms": fn_one_ms,
                                "one_pass_extra_ms": fn_one_ms - stage_mean("probe_attention")},
            "hkvd_selector": {"ms": hk_ms, "algorithmic_gb": hk_gb, "gbs": hk_gb / (hk_ms * 1e-3),
                              "requests_timed": hk_nb, "timed_calls_gbs": hk_timed_gbs},
        }
    fp = A.acache_kv_footprint([w.T] * w.batch, w.L, S.K, w.page_size, w.n_layers, w.n_kv_heads, w.head_dim, w.dtype)
    stage_t = {name: [evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)]
               for j, name in enumerate(Setup.STAGES)}
    stage_ms = {name: float(np.mean(t)) for name, t in stage_t.items()}
    stage_pct = {q: {name: float(np.percentile(t, q)) for name, t in stage_t.items()} for q in (10, 50, 90)}
    wm = work_model(w, S.K)
    t_map = stage_ms["mapped_attention"] * 1e-3
    t_probe = stage_ms["probe_attention"] * 1e-3
    mapped_tflops = wm["mapped_flops"] / t_map / 1e12
    probe_ms_req = (stage_ms["probe_attention"] + stage_ms["probe_column_mass"] + stage_ms["topk_maps"]) / w.batch
    probe_tflops = wm["probe_flops"] / t_probe / 1e12
    traffic = measured_traffic(w.name)
    probe_k = many_query_kernel(w.n_q_heads, w.n_kv_heads, S.n_rows)
    roof = {"kernel": f"{probe_k} (probe attention, one launch for all layers)", "bound": "mfma",
            "achieved": probe_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": probe_tflops / PEAK_BF16_TFLOPS, "traffic": traffic.get(probe_k),
            "traffic_unit": "HBM bytes per launch", "algorithmic_per_launch": wm["probe_flops"],
            "algorithmic_bytes_per_launch": wm["probe_bytes"]}
    mapped_gbs = wm["mapped_bytes"] / t_map / 1e9
    # grouped query heads raise the read-slot attention's intensity past the
    # ridge (2.5 PFLOP/s over 8 TB/s): it is then bound by the matrix units
    mapped_mfma = wm["mapped_flops"] / wm["mapped_bytes"] > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if mapped_mfma:
        map_kernels = (many_query_kernel(w.n_q_heads, w.n_kv_heads, w.block_len),)   # packed query-head groups
        roof_kernel = f"read-slot attention, one call for all layers ({map_kernels[0]}, query-head groups packed)"
    elif w.batch < 2:
        # one request shares the affix with no other: the shared-affix call runs the single pass
        map_kernels = ("attn_split_mfma",)
        roof_kernel = "read-slot attention, one shared-affix call for all layers (single pass: attn_split_mfma)"
    else:
        map_kernels = ("shared_plan_kernel", "attn_shared_mfma")
        roof_kernel = "read-slot attention, one shared-affix call for all layers (" + " + ".join(map_kernels) + ")"
    map_traffic = [traffic.get(k) for k in map_kernels]
    roof_mapped = {"kernel": roof_kernel, "bound": "mfma" if mapped_mfma else "hbm",
                   "achieved": mapped_tflops if mapped_mfma else mapped_gbs,
                   "peak": PEAK_BF16_TFLOPS if mapped_mfma else PEAK_HBM_GBS,
                   "unit": "TFLOP/s" if mapped_mfma else "GB/s",
                   "frac": mapped_tflops / PEAK_BF16_TFLOPS if mapped_mfma else mapped_gbs / PEAK_HBM_GBS,
                   "traffic": sum(map_traffic) if all(t is not None for t in map_traffic) else None,
                   "traffic_unit": "HBM bytes per call", "algorithmic_per_launch":
                   wm["mapped_flops"] if mapped_mfma else wm["mapped_bytes"],
                   "algorithmic_bytes_per_launch": wm["mapped_bytes"], "algorithmic_gbs": mapped_gbs}
    scatter_gbs = wm["scatter_bytes"] / (stage_ms["admission_scatter"] * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": mapped_tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": total_ms / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "layers": w.n_layers, "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "affix_L": w.L, "affix_at": w.affix_l, "request_tokens": w.P - w.m,
                   "gen_tokens": w.m, "batch": w.batch, "anchor_rate": w.rate, "K": S.K, "decode_block": w.block_len,
                   "logical_len": w.T, "page_size": w.page_size, "page_order": w.page_order,
                   "shared_slot_order": w.shared_slot_order},
        "mapped_attention_pct_bf16_peak": 100.0 * mapped_tflops / PEAK_BF16_TFLOPS,
        "kv_footprint_gb": {"shared": fp["shared"] / 1e9, "private": fp["private"] / 1e9,
                            "dense": fp["dense"] / 1e9,
                            "acache_saving": 1 - (fp["shared"] + fp["private"]) / fp["dense"]},
        "probe_ms_per_request": probe_ms_req,
        "probe_attention_tflops": probe_tflops,
        # the probe's algorithmic bytes (affix K/V once, Q, O_aff, LSE) over its time: with few rows per request
        # (one request at L=1024) the probe sits near the ridge, so both fractions are reported
        "probe_attention_hbm": {"achieved": wm["probe_bytes"] / t_probe / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": wm["probe_bytes"] / t_probe / 1e9 / PEAK_HBM_GBS,
                                "algorithmic_bytes_per_launch": wm["probe_bytes"]},
        "admission_scatter_gbs": scatter_gbs,
        "stage_ms": stage_ms,
        "stage_ms_p10": stage_pct[10],
        "stage_ms_median": stage_pct[50],
        "stage_ms_p90": stage_pct[90],
        "roofline": roof,
        "roofline_mapped": roof_mapped,
    }
    out.update(extras)
    if args.ceilings:
        out["library_ceilings"] = library_ceilings(w, dev)
    if host is not None:
        out["cpu_baseline"] = cpu_baseline(w, S, host)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
