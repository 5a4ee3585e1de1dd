"""Plain fp64 CPU oracle for the ACache slot-mapped attention engine.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never imports or calls it, and this
module imports nothing from the product path.

Source: "Affix Cache for Diffusion Large Language Models" (ACache), arXiv
2608.26140.  Every function states the passage it follows.  Each one is
written for a reader to check against the paper by eye: explicit per-slot
gathers, one (layer, head) at a time, a numpy matmul as the only library
primitive for the dot products, no blocking or fusion.

Readings taken where the paper leaves a step open (all listed in the
design notes with their reasons):
  * Eq. (4) normalises over the affix keys only (its softmax argument is
    Q_mask K_affix^T), so every masked row's affix mass sums to one.
  * The probe forms O_aff and LSE_aff for every non-affix row (the probe
    forward, cost O(N H P L) in Section 3.2); only the initially masked rows
    contribute to s_j.
  * Heads are query heads; under grouped-query attention query head h reads
    KV head h // (Hq / Hkv).
  * K = ceil(rate * L) (with a 1e-9 guard), clamped to [0, L].
  * Top-K ties go to the lower affix offset; anchors are returned as
    ascending logical positions.
  * Private slot i of a request is assigned in ascending logical order of
    the recompute set R = A u (non-affix positions).

Pins.  Every function here is checked against something other than itself
(hand-worked fixtures, closed forms, library routines on special cases, a
pure-Python brute force; see the oracle tests).  Three readings of the paper
stay parity unpinned against the paper itself, because it prints no value
that decides them: the affix-only normaliser of Eq. (4) (probe_layer; the
full-context alternative is probe_layer_full), ceil rather than round in
anchor_count (they differ at L = 4096 and 16384), and the squared-L2 reduction
of the KV difference in hkvd_scores.  Each function is pinned to the
mathematics of its reading.
"""
import math
import numpy as np


# ----------------------------------------------------------------------------
# input decoding (bf16 bit patterns or fp32 values -> fp64, exactly)
# ----------------------------------------------------------------------------
def decode(x):
    """fp64 view of stored values.  uint16/int16 arrays are bf16 bit patterns:
    a bf16 number is the upper half of the fp32 with the same bits, so the
    widening is exact."""
    x = np.asarray(x)
    if x.dtype in (np.uint16, np.int16):
        u = x.view(np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)
    return x.astype(np.float64)


# ----------------------------------------------------------------------------
# anchor count (Section 5, Default Settings: anchor ratios {0, .1, .2, .3, .5, 1})
# ----------------------------------------------------------------------------
def anchor_count(L, rate):
    """Number of Anchor Tokens for an affix of L tokens at anchor ratio `rate`:
    ceil(rate * L), guarded against rate*L landing a hair above an integer,
    clamped to [0, L].  Rate 0 is direct reuse, rate 1 full recomputation
    (Section 5.1)."""
    if not (0.0 <= rate <= 1.0):
        raise ValueError("rate must lie in [0, 1]")
    k = math.ceil(rate * L - 1e-9)
    return max(0, min(L, k))


# ----------------------------------------------------------------------------
# paged KV access (Section 4.1: paged physical slots; slot s = page s // ps,
# offset s % ps)
# ----------------------------------------------------------------------------
def slot_rows(pool_layer, slots, kv_head, page_size):
    """Gather one KV head's rows for a list of physical slots: row i is
    pool_layer[page(slots[i]), kv_head, offset(slots[i])], in the order of
    `slots`.  pool_layer: [n_pages][Hkv][page_size][d] (stored values)."""
    slots = np.asarray(slots, np.int64)
    return decode(pool_layer[slots // page_size, kv_head, slots % page_size])


def kv_head_of(h, n_q_heads, n_kv_heads):
    return h // (n_q_heads // n_kv_heads)


def softmax_rows(S):
    """Row softmax with its log-sum-exp; returns (P, lse)."""
    m = S.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(S - m).sum(axis=1))
    return np.exp(S - lse[:, None]), lse


# ----------------------------------------------------------------------------
# one-shot anchor probe: Section 3.2, Eqs. (4) and (5)
# ----------------------------------------------------------------------------
def probe_layer(q_layer, k_layer, v_layer, shared_slots, page_size, n_kv_heads,
                masked_rows, masked_offsets, scale, want_out=True):
    """One layer of the probe.

    q_layer: [rows][Hq][d] queries of every non-affix row of the batch.
    k_layer, v_layer: [n_pages][Hkv][ps][d] pool of this layer.
    shared_slots: [L] physical slot of affix offset j (the shared region).
    masked_rows / masked_offsets: rows of request b that were masked at the
    start (M_T) are masked_rows[masked_offsets[b]:masked_offsets[b+1]].

    Returns O_aff [rows][Hq][d], LSE_aff [rows][Hq] (natural log) and the
    layer's contribution to s_j, [B][L]: sum over query heads and masked rows
    of the Eq. (4) weights a_{j,k} = softmax_j(q_k . k_j * scale).
    """
    rows, Hq, d = q_layer.shape
    L = len(shared_slots)
    B = len(masked_offsets) - 1
    o = np.zeros((rows, Hq, d)) if want_out else None
    lse = np.zeros((rows, Hq))
    s = np.zeros((B, L))
    for h in range(Hq):
        g = kv_head_of(h, Hq, n_kv_heads)
        Kaff = slot_rows(k_layer, shared_slots, g, page_size)      # [L][d]
        Q = decode(q_layer[:, h, :])                                  # [rows][d]
        A, lse[:, h] = softmax_rows((Q @ Kaff.T) * scale)             # Eq. (4), every probe row
        if want_out:
            o[:, h, :] = A @ slot_rows(v_layer, shared_slots, g, page_size)
        for b in range(B):
            mk = masked_rows[masked_offsets[b]:masked_offsets[b + 1]]
            s[b] += A[mk].sum(axis=0)                                  # Eq. (5): sum over k in M_T
    return o, lse, s


def probe_scores(q, k_pool, v_pool, shared_slots, page_size, n_kv_heads, masked_rows,
                 masked_offsets, scale):
    """Eq. (5) over all layers: s_j = sum_n sum_h sum_{k in M_T} a^{(n,h)}_{j,k}.
    q: [N][rows][Hq][d]; pools [N][n_pages][Hkv][ps][d].  Returns [B][L]."""
    B = len(masked_offsets) - 1
    s = np.zeros((B, len(shared_slots)))
    for n in range(q.shape[0]):
        _, _, sn = probe_layer(q[n], k_pool[n], v_pool[n], shared_slots, page_size, n_kv_heads,
                               masked_rows, masked_offsets, scale, want_out=False)
        s += sn
    return s


# ----------------------------------------------------------------------------
# Top-K anchor set: Section 3.2, Eq. (6)
# ----------------------------------------------------------------------------
def topk_anchors(scores_b, K, affix_l):
    """A = TopK({s_j}, K): the K affix offsets of largest score (ties to the
    lower offset), returned as ascending logical positions l + j.
    The non-anchor set S = F \\ A is everything else in the span."""
    scores_b = np.asarray(scores_b)
    order = np.lexsort((np.arange(len(scores_b)), -scores_b))   # score desc, then offset asc
    return np.sort(order[:K]).astype(np.int64) + affix_l


# ----------------------------------------------------------------------------
# the two per-request maps: Section 4.1 (KV Layout and Dual Mapping) and
# Section 4.2 (Admission-Time Preparation)
# ----------------------------------------------------------------------------
def build_maps(anchors_b, T, affix_l, L, shared_slots, private_pages_b, page_size):
    """Write-side recomputation map and read-slot map of one request.

    R = anchors u non-affix positions, in ascending logical order; its i-th
    member gets private slot private_pages_b[i // ps] * ps + i % ps.
    read_slot[p] = shared_slots[p - l] for a non-anchor affix position,
    else the private slot of p.
    Returns (read_slot [T], recompute_pos [R], recompute_slot [R])."""
    anchors = set(int(a) for a in anchors_b)
    read_slot = np.full(T, -1, np.int64)
    rc_pos, rc_slot = [], []
    for p in range(T):
        in_affix = affix_l <= p < affix_l + L
        if in_affix and p not in anchors:
            read_slot[p] = shared_slots[p - affix_l]
            continue
        i = len(rc_pos)
        slot = int(private_pages_b[i // page_size]) * page_size + i % page_size
        rc_pos.append(p)
        rc_slot.append(slot)
        read_slot[p] = slot
    return read_slot, np.array(rc_pos, np.int64), np.array(rc_slot, np.int64)


# ----------------------------------------------------------------------------
# write-side scatter: Section 4.3, Appendix C.1 (store-then-attend: new KV is
# written through the write-side slot mapping first)
# ----------------------------------------------------------------------------
def scatter(k_pool, v_pool, k_src, v_src, dst_slots, page_size):
    """pool[n][slot dst[i]] = src[n][i] for every layer n and KV head, one row
    at a time.  Pools are modified in place (pass copies)."""
    for n in range(k_src.shape[0]):
        for i, s in enumerate(dst_slots):
            s = int(s)
            k_pool[n, s // page_size, :, s % page_size, :] = k_src[n, i]
            v_pool[n, s // page_size, :, s % page_size, :] = v_src[n, i]


# ----------------------------------------------------------------------------
# read-slot attention: Section 4.3 (Online Inference Loop) and Appendix C.1
# ----------------------------------------------------------------------------
def mapped_attention_layer(q_layer, k_layer, v_layer, q_offsets, read_slot, kv_offsets,
                           n_kv_heads, page_size, scale):
    """Bidirectional attention of request b's query rows over every logical
    position 0..T_b-1, whose key and value are read at physical slot
    read_slot[kv_offsets[b] + p].
    q_layer [n_q][Hq][d]; returns O [n_q][Hq][d] and LSE [n_q][Hq].
    A request with no logical positions (T_b = 0) attends over an empty set:
    its weighted sum is empty (O = 0) and its log-sum-exp is log 0 = -inf."""
    n_q, Hq, d = q_layer.shape
    o = np.zeros((n_q, Hq, d))
    lse = np.zeros((n_q, Hq))
    for b in range(len(q_offsets) - 1):
        q0, q1 = q_offsets[b], q_offsets[b + 1]
        slots = read_slot[kv_offsets[b]:kv_offsets[b + 1]]
        if q1 == q0:
            continue
        if len(slots) == 0:
            lse[q0:q1, :] = -np.inf
            continue
        for h in range(Hq):
            g = kv_head_of(h, Hq, n_kv_heads)
            Kl = slot_rows(k_layer, slots, g, page_size)      # [T_b][d], logical order
            Vl = slot_rows(v_layer, slots, g, page_size)
            Q = decode(q_layer[q0:q1, h, :])
            A, lse[q0:q1, h] = softmax_rows((Q @ Kl.T) * scale)
            o[q0:q1, h, :] = A @ Vl
    return o, lse


def block_slots(read_slot, kv_offsets, block_start, block_len):
    """Destination slots of a decode block: request b's positions
    block_start[b] .. +block_len, read through its read-slot map (Section 4.3,
    Block decoding: the block's KV goes to the slots the map names)."""
    out = []
    for b in range(len(kv_offsets) - 1):
        for i in range(block_len):
            out.append(int(read_slot[kv_offsets[b] + block_start[b] + i]))
    return np.array(out, np.int64)


# ----------------------------------------------------------------------------
# DropNA ablation (Section 5.3, Figure 5): same Anchor Tokens, the non-anchor
# affix cache discarded
# ----------------------------------------------------------------------------
def dropna_read_table(read_slot_b, anchors_b, affix_l, L):
    """Read list of one request under DropNA: its KeepNA read-slot list with
    every non-anchor affix position (p in F \\ A) left out, in logical
    order.  Anchors and all positions outside the affix keep their slots."""
    anchor_set = set(int(a) for a in anchors_b)
    keep = []
    for p in range(len(read_slot_b)):
        in_affix = affix_l <= p < affix_l + L
        if in_affix and p not in anchor_set:
            continue
        keep.append(int(read_slot_b[p]))
    return np.array(keep, np.int64)


# ----------------------------------------------------------------------------
# KV-cache footprint of the two layouts (Section 4.1 shared/private regions,
# Appendix B.2: blocks are allocated per region at block granularity)
# ----------------------------------------------------------------------------
def kv_footprint(seq_len, L, K, page_size, slot_bytes):
    """Peak KV bytes with every request of the batch resident.

    dense:   each request holds its whole logical context in its own pages
             (the baseline cache, no sharing);
    shared:  the affix is stored once, in ceil(L / ps) shared pages;
    private: each request holds its recompute set R_b = K + (T_b - L)
             (anchors and request positions) in ceil(R_b / ps) pages;
    dropna:  the private pages alone (the non-anchor affix cache dropped).
    slot_bytes = K and V bytes of one slot over all layers and KV heads."""
    pages = lambda n: -(-int(n) // page_size)
    dense = sum(pages(t) for t in seq_len) * page_size * slot_bytes
    shared = pages(L) * page_size * slot_bytes if len(seq_len) else 0
    private = sum(pages(K + t - L) for t in seq_len) * page_size * slot_bytes
    return {"dense": dense, "shared": shared, "private": private, "acache": shared + private,
            "dropna": private}


# ----------------------------------------------------------------------------
# Full-context reading of the probe normaliser (the alternative to Eq. (4)
# read literally): each non-affix row's softmax runs over the affix keys AND
# the request's own non-affix keys; the scores still sum only affix weights
# ----------------------------------------------------------------------------
def probe_layer_full(q_layer, k_layer, v_layer, shared_slots, row_offsets, na_slots, na_offsets,
                     page_size, n_kv_heads, masked_rows, masked_offsets, scale):
    """One layer of the probe with the full-context normaliser.

    Request b's non-affix rows are q rows row_offsets[b]..row_offsets[b+1];
    its non-affix keys and values sit at slots na_slots[na_offsets[b] ..
    na_offsets[b+1]].  Each row attends over [affix keys, own non-affix keys]
    in one softmax.  Returns O [rows][Hq][d], LSE [rows][Hq] (natural log)
    and the layer's [B][L] sum of the affix weights over heads and the masked
    rows of each request (masked_rows index the batch's rows)."""
    rows, Hq, d = q_layer.shape
    L = len(shared_slots)
    B = len(row_offsets) - 1
    o = np.zeros((rows, Hq, d))
    lse = np.zeros((rows, Hq))
    s = np.zeros((B, L))
    for b in range(B):
        r0, r1 = row_offsets[b], row_offsets[b + 1]
        own = na_slots[na_offsets[b]:na_offsets[b + 1]]
        mk = masked_rows[masked_offsets[b]:masked_offsets[b + 1]] - r0     # masked rows of b, local index
        for h in range(Hq):
            g = kv_head_of(h, Hq, n_kv_heads)
            Kc = np.concatenate([slot_rows(k_layer, shared_slots, g, page_size),
                                 slot_rows(k_layer, own, g, page_size)])
            Vc = np.concatenate([slot_rows(v_layer, shared_slots, g, page_size),
                                 slot_rows(v_layer, own, g, page_size)])
            Q = decode(q_layer[r0:r1, h, :])
            A, lse[r0:r1, h] = softmax_rows((Q @ Kc.T) * scale)
            o[r0:r1, h, :] = A @ Vc
            s[b] += A[mk, :L].sum(axis=0)
    return o, lse, s


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Attention over the union of two disjoint key sets from the attentions
    over each (their outputs and natural-log log-sum-exps): the softmax over
    the union weights each part by its share of the total exponential mass.
    Two empty parts give O = 0 and LSE = -inf."""
    lse = np.logaddexp(lse_a, lse_b)
    wa = np.where(np.isneginf(lse), 0.0, np.exp(lse_a - np.where(np.isneginf(lse), 0.0, lse)))
    wb = np.where(np.isneginf(lse), 0.0, np.exp(lse_b - np.where(np.isneginf(lse), 0.0, lse)))
    return wa[..., None] * o_a + wb[..., None] * o_b, lse


# ----------------------------------------------------------------------------
# CacheBlend-style HKVD selector (Appendix B.5): rank affix tokens by how far
# their full-prompt KV lies from the affix-only (shared) cache
# ----------------------------------------------------------------------------
def hkvd_scores(k_pool, v_pool, shared_slots, k_full, v_full, page_size):
    """Per request b and affix offset j: the squared L2 norm of the
    difference between the token's full-prompt K and V (k_full / v_full
    [N][B][L][Hkv][d]) and its affix-only K and V in the shared region (pool
    slot shared_slots[j]), summed over layers, KV heads, K and V.  Its Top-K
    is the Top-K of the norm itself.  Returns [B][L]."""
    N, B, L, Hkv, d = k_full.shape
    s = np.zeros((B, L))
    for n in range(N):
        for g in range(Hkv):
            Ka = slot_rows(k_pool[n], shared_slots, g, page_size)      # [L][d]
            Va = slot_rows(v_pool[n], shared_slots, g, page_size)
            for b in range(B):
                dk = decode(k_full[n, b, :, g, :]) - Ka
                dv = decode(v_full[n, b, :, g, :]) - Va
                s[b] += (dk * dk).sum(axis=1) + (dv * dv).sum(axis=1)
    return s
