"""Seeded synthetic inputs for the slot-mapped attention engine.

Everything here is *input*: the physical page allocation a serving engine
would hand over (shared pages holding the affix, per-request private pages,
free pages), and seeded random Q/K/V tensors.  Values follow one recipe:

* Q, K, V ~ N(0, 1), generated in fp32 and rounded once to the storage type
  (bf16 round-to-nearest-even via torch's cast).
* "sinks": a seeded set of affix offsets whose keys are scaled by 4 in every
  layer and KV head (concentrates attention mass, as the stable high-mass
  affix positions of the paper's Figure 2 motivate).
* "heavy": a seeded 1% of affix offsets whose keys are Student-t (nu = 3),
  drawn as z0 / sqrt((z1^2 + z2^2 + z3^2) / 3).
* recomputed rows for the private scatter ~ N(0, 1).

Nothing in this module computes anything the method computes: the anchor
count, the top-K, the slot maps and every attention quantity are produced
separately by the library under test and by the oracle.  The generator only
needs the anchor count K to size each request's private region (K + P slots).
"""
from dataclasses import dataclass
import numpy as np
import torch

from .configs import Workload

# stream ids of the seed tree
S_PAGES, S_POOL_K, S_POOL_V, S_QPROBE, S_TWEAK, S_SRC_K, S_SRC_V, S_QDEC, S_BLK_K, S_BLK_V, S_SCORES, S_QRC = range(12)

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def seed_of(base, cid, stream, *ids):
    ss = np.random.SeedSequence([int(base), int(cid), int(stream)] + [int(i) for i in ids])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)


def _randn(shape, seed, device, dtype):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.to(dtype)


@dataclass
class Layout:
    """Physical page allocation and ragged-batch offsets (host numpy, int32)."""
    n_pages: int
    page_owner: np.ndarray          # [n_pages]: -1 shared, b = request b's private page, -2 free
    shared_pages: np.ndarray        # [ceil(L/ps)]
    shared_slots: np.ndarray        # [L]: affix offset j -> physical slot
    private_pages: np.ndarray       # flat, request b at private_page_offsets[b]..[b+1]
    private_page_offsets: np.ndarray  # [B+1]
    seq_len: np.ndarray             # [B] logical length T_b
    kv_offsets: np.ndarray          # [B+1] prefix sums of T_b (read-slot table offsets)
    rc_offsets: np.ndarray          # [B+1] prefix sums of K + P_b (recompute table offsets)
    probe_pos: np.ndarray           # [B*P]: logical position of each probe row (non-affix)
    row_offsets: np.ndarray         # [B+1] probe rows per request
    masked_rows: np.ndarray         # [B*m]: probe-row index of each initially masked row
    masked_offsets: np.ndarray      # [B+1]


def make_layout(w: Workload, K: int, seed: int = 0, page_order=None, shared_slot_order=None) -> Layout:
    ps, B, L, P, T = w.page_size, w.batch, w.L, w.P, w.T
    page_order = page_order or w.page_order
    shared_slot_order = shared_slot_order or w.shared_slot_order
    R = K + P
    n_shared = -(-L // ps)
    n_priv = -(-R // ps)
    used = n_shared + B * n_priv
    rng = np.random.default_rng(seed_of(seed, w.cid, S_PAGES))
    if page_order == "identity":
        n_pages = used
        phys = np.arange(n_pages)
    elif page_order == "random":
        n_pages = used
        phys = rng.permutation(n_pages)
    elif page_order == "fragmented":
        n_pages = int(np.ceil(used / (1.0 - w.free_frac)))
        phys = rng.permutation(n_pages)
    else:
        raise ValueError(page_order)
    owner = np.full(n_pages, -2, np.int32)
    shared_pages = phys[:n_shared].astype(np.int32)
    owner[shared_pages] = -1
    priv = []
    for b in range(B):
        pg = phys[n_shared + b * n_priv: n_shared + (b + 1) * n_priv]
        owner[pg] = b
        priv.append(pg)
    private_pages = np.concatenate(priv).astype(np.int32)
    private_page_offsets = (np.arange(B + 1) * n_priv).astype(np.int32)
    all_shared = (shared_pages[:, None] * ps + np.arange(ps)[None, :]).reshape(-1)
    if shared_slot_order == "page":
        shared_slots = all_shared[:L]
    elif shared_slot_order == "slot":
        shared_slots = rng.permutation(all_shared)[:L]
    else:
        raise ValueError(shared_slot_order)
    seq_len = np.full(B, T, np.int32)
    kv_offsets = np.concatenate([[0], np.cumsum(seq_len)]).astype(np.int32)
    rc_offsets = (np.arange(B + 1) * R).astype(np.int32)
    na = np.array(w.non_affix_positions(), np.int32)
    probe_pos = np.tile(na, B).astype(np.int32)
    row_offsets = (np.arange(B + 1) * P).astype(np.int32)
    gen = set(w.positions("gen"))
    local_masked = np.array([i for i, p in enumerate(na) if p in gen], np.int32)
    masked_rows = np.concatenate([b * P + local_masked for b in range(B)]).astype(np.int32)
    masked_offsets = (np.arange(B + 1) * len(local_masked)).astype(np.int32)
    return Layout(n_pages, owner, shared_pages, shared_slots.astype(np.int32), private_pages,
                  private_page_offsets, seq_len, kv_offsets, rc_offsets, probe_pos, row_offsets,
                  masked_rows, masked_offsets)


def tweak_offsets(w: Workload, seed: int = 0):
    """Affix offsets that carry sink keys (x4) or heavy-tailed keys."""
    rng = np.random.default_rng(seed_of(seed, w.cid, S_TWEAK))
    if w.key_tweak == "sinks":
        return np.sort(rng.choice(w.L, size=min(w.n_sinks, w.L), replace=False)).astype(np.int64)
    if w.key_tweak == "heavy":
        n = max(1, int(round(w.heavy_frac * w.L)))
        return np.sort(rng.choice(w.L, size=n, replace=False)).astype(np.int64)
    return np.zeros(0, np.int64)


def make_pool(w: Workload, lay: Layout, device="cpu", seed: int = 0, layers=None):
    """K and V pools [n_layers][n_pages][Hkv][ps][d]; every page holds N(0,1)
    content, and the shared pages hold the affix K/V (with the key tweak)."""
    dt = TORCH_DT[w.dtype]
    layers = range(w.n_layers) if layers is None else layers
    nl = len(layers)
    shape = (lay.n_pages, w.n_kv_heads, w.page_size, w.head_dim)
    k = torch.empty((nl,) + shape, dtype=dt, device=device)
    v = torch.empty((nl,) + shape, dtype=dt, device=device)
    offs = tweak_offsets(w, seed)
    slots = torch.as_tensor(lay.shared_slots[offs].astype(np.int64), device=device)
    pg, off = slots // w.page_size, slots % w.page_size
    for i, n in enumerate(layers):
        k[i] = _randn(shape, seed_of(seed, w.cid, S_POOL_K, n), device, dt)
        v[i] = _randn(shape, seed_of(seed, w.cid, S_POOL_V, n), device, dt)
        if len(offs) == 0:
            continue
        if w.key_tweak == "sinks":
            rows = k[i][pg, :, off, :].float() * w.sink_scale
            k[i][pg, :, off, :] = rows.to(dt)
        elif w.key_tweak == "heavy":
            z = _randn((4, len(offs), w.n_kv_heads, w.head_dim),
                       seed_of(seed, w.cid, S_TWEAK, 1, n), device, torch.float32)
            t = z[0] / torch.sqrt((z[1] ** 2 + z[2] ** 2 + z[3] ** 2) / w.heavy_nu)
            k[i][pg, :, off, :] = t.to(dt)
    return k, v


def make_probe_q(w: Workload, lay: Layout, device="cpu", seed: int = 0, layers=None):
    dt = TORCH_DT[w.dtype]
    layers = range(w.n_layers) if layers is None else layers
    rows = len(lay.probe_pos)
    q = torch.empty((len(layers), rows, w.n_q_heads, w.head_dim), dtype=dt, device=device)
    for i, n in enumerate(layers):
        q[i] = _randn(q.shape[1:], seed_of(seed, w.cid, S_QPROBE, n), device, dt)
    return q


def make_rows(w: Workload, n_rows: int, stream: int, device="cpu", seed: int = 0, layers=None,
              heads=None, step: int = 0):
    """[n_layers][n_rows][heads][d] of N(0,1): recomputed K/V rows, decode Q,
    recompute-phase Q."""
    dt = TORCH_DT[w.dtype]
    layers = range(w.n_layers) if layers is None else layers
    heads = w.n_kv_heads if heads is None else heads
    x = torch.empty((len(layers), n_rows, heads, w.head_dim), dtype=dt, device=device)
    for i, n in enumerate(layers):
        x[i] = _randn(x.shape[1:], seed_of(seed, w.cid, stream, n, step), device, dt)
    return x


def block_positions(w: Workload, step: int):
    """Logical positions of decode block `step` (the step-th block of the
    generation span), identical for every request."""
    g0 = w.gen_start()
    return list(range(g0 + step * w.block_len, g0 + (step + 1) * w.block_len))


def seeded_scores(w: Workload, seed: int = 0, device="cpu"):
    """Random non-negative per-affix scores [B][L] (for Top-K tests only)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(seed, w.cid, S_SCORES))
    return torch.rand((w.batch, w.L), generator=g, device=device, dtype=torch.float32)


def to_device_i32(a, device):
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32), device=device)
