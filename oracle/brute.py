"""Brute-force pure-Python re-statement of the oracle, for tiny inputs.

TEST INFRASTRUCTURE ONLY (same rule as acache_oracle: only tests, the smoke
check and the CPU-baseline leg may use it).  It shares no code with
acache_oracle: scalar loops over Python floats with math.exp, a rank-count
Top-K instead of a sort, and a closed-form private index instead of a scan,
so that a slip in one formulation shows up as a disagreement with the other.
Source: "Affix Cache for Diffusion Large Language Models", Section 3.2
(Eqs. 4-6), Section 4.1-4.3 and Appendix C.1.
"""
import math
import struct


def _val(x):
    """Python float from a stored element (numpy scalar, int bf16 bits)."""
    if hasattr(x, "dtype") and str(x.dtype) in ("uint16", "int16"):
        bits = (int(x) & 0xFFFF) << 16
        return struct.unpack("<f", struct.pack("<I", bits))[0]
    return float(x)


def _row(pool_layer, slot, g, ps):
    return [_val(e) for e in pool_layer[slot // ps][g][slot % ps]]


def _dot(a, b):
    t = 0.0
    for x, y in zip(a, b):
        t += x * y
    return t


def _attend(q, keys, vals, scale):
    logits = [_dot(q, k) * scale for k in keys]
    mx = max(logits)
    w = [math.exp(z - mx) for z in logits]
    tot = sum(w)
    p = [x / tot for x in w]
    d = len(vals[0])
    o = [sum(p[j] * vals[j][c] for j in range(len(vals))) for c in range(d)]
    return p, o, mx + math.log(tot)


def probe(q, k_pool, v_pool, shared_slots, ps, n_kv, masked_rows, masked_offsets, scale):
    """Returns (scores [B][L], O_aff [N][rows][Hq][d], LSE [N][rows][Hq]) as lists."""
    N, rows, Hq = len(q), len(q[0]), len(q[0][0])
    B, L = len(masked_offsets) - 1, len(shared_slots)
    grp = Hq // n_kv
    scores = [[0.0] * L for _ in range(B)]
    O = [[[None] * Hq for _ in range(rows)] for _ in range(N)]
    LSE = [[[0.0] * Hq for _ in range(rows)] for _ in range(N)]
    masked_owner = {}
    for b in range(B):
        for i in range(masked_offsets[b], masked_offsets[b + 1]):
            masked_owner[int(masked_rows[i])] = b
    for n in range(N):
        for h in range(Hq):
            g = h // grp
            keys = [_row(k_pool[n], int(s), g, ps) for s in shared_slots]
            vals = [_row(v_pool[n], int(s), g, ps) for s in shared_slots]
            for r in range(rows):
                qv = [_val(e) for e in q[n][r][h]]
                p, o, lse = _attend(qv, keys, vals, scale)
                O[n][r][h] = o
                LSE[n][r][h] = lse
                if r in masked_owner:
                    b = masked_owner[r]
                    for j in range(L):
                        scores[b][j] += p[j]
    return scores, O, LSE


def topk(scores_b, K, affix_l):
    """Offset j is an anchor iff fewer than K offsets beat it (higher score,
    or equal score at a lower offset)."""
    L = len(scores_b)
    out = []
    for j in range(L):
        beats = 0
        for i in range(L):
            if scores_b[i] > scores_b[j] or (scores_b[i] == scores_b[j] and i < j):
                beats += 1
        if beats < K:
            out.append(affix_l + j)
    return out


def maps(anchors, T, affix_l, L, shared_slots, private_pages, ps):
    """Closed-form private index: positions before the affix keep their
    position, anchor number r (ascending) gets l + r, positions after the
    affix get p - L + K."""
    K = len(anchors)
    rank = {a: r for r, a in enumerate(sorted(anchors))}
    read_slot = []
    rc = []
    for p in range(T):
        if p < affix_l:
            i = p
        elif p < affix_l + L:
            if p not in rank:
                read_slot.append(int(shared_slots[p - affix_l]))
                continue
            i = affix_l + rank[p]
        else:
            i = p - L + K
        slot = int(private_pages[i // ps]) * ps + i % ps
        read_slot.append(slot)
        rc.append((i, p, slot))
    rc.sort()
    return read_slot, [p for _, p, _ in rc], [s for _, _, s in rc]


def mapped_attention(q, k_pool, v_pool, q_offsets, read_slot, kv_offsets, n_kv, ps, scale):
    """O [N][n_q][Hq][d] as lists."""
    N, n_q, Hq = len(q), len(q[0]), len(q[0][0])
    grp = Hq // n_kv
    O = [[[None] * Hq for _ in range(n_q)] for _ in range(N)]
    for n in range(N):
        for b in range(len(q_offsets) - 1):
            slots = [int(s) for s in read_slot[kv_offsets[b]:kv_offsets[b + 1]]]
            for h in range(Hq):
                g = h // grp
                keys = [_row(k_pool[n], s, g, ps) for s in slots]
                vals = [_row(v_pool[n], s, g, ps) for s in slots]
                for r in range(q_offsets[b], q_offsets[b + 1]):
                    _, o, _ = _attend([_val(e) for e in q[n][r][h]], keys, vals, scale)
                    O[n][r][h] = o
    return O


def block_slots(anchors, affix_l, L, private_pages, ps, block_start, block_len):
    """Destination slots of each request's decode block, from the closed-form
    private index of maps() (no read-slot table): request b's positions
    block_start[b] .. +block_len, in request order.  anchors[b] and
    private_pages[b] are request b's own lists.  Decode blocks lie outside
    the affix or on anchors (private positions); a non-anchor affix position
    is refused."""
    out = []
    for b in range(len(block_start)):
        K = len(anchors[b])
        rank = {a: r for r, a in enumerate(sorted(anchors[b]))}
        for p in range(block_start[b], block_start[b] + block_len):
            if p < affix_l:
                i = p
            elif p < affix_l + L:
                if p not in rank:
                    raise ValueError("a decode block inside the affix reads the shared region")
                i = affix_l + rank[p]
            else:
                i = p - L + K
            out.append(int(private_pages[b][i // ps]) * ps + i % ps)
    return out
