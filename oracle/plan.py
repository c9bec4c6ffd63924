"""Plain numpy twin of the quartet plan -- TEST INFRASTRUCTURE ONLY.

The page (FusionRCG, section III-C and section V) batches shell quartets per
angular-momentum class ("shell-quartet classes", 120 of them for l <= 4 per
section IV "Build system") and relies on the 8-fold permutation symmetry of
(ab|cd) (section III-C2, Kernel 2).  It prints no canonical form, sort key
or screening rule.  Readings taken (the HIP library implements the same
rules independently):

* pair class pc(la, lb) = la(la+1)/2 + lb for la >= lb; quartet class
  id = pcb(pcb+1)/2 + pck for pcb >= pck.  l <= 4 gives 15 pair classes and
  120 quartet classes.
* canonical quartet: swap within the bra so that l_a >= l_b (bit 0), within
  the ket so that l_c >= l_d (bit 1), then bra with ket if pc(bra) < pc(ket)
  (bit 2).  The 3-bit code is stored with the quartet.
* explicit lists are ordered by (class id, K_bra, K_ket, input position),
  where K_bra = K_a K_b is the primitive-pair count.
* screened lists: pairs i >= j (pair index i(i+1)/2 + j) oriented so that
  l_a >= l_b; each pair belongs to the bucket (pc, K_pair); inside a bucket
  pairs are ranked by Schwarz factor descending, ties by pair index.  For
  two pairs p, q the bra is the one in the later bucket (buckets ordered by
  (pc, K)), or the lower rank in the same bucket; (p, q) survives iff
  fl(S_p * S_q) >= fl(tau * tau).  Order: (class id, K_bra, K_ket, bra rank,
  ket rank).  The Schwarz factor itself is S_ij = max |(mu nu|mu nu)| over
  the (ij|ij) block (the caller supplies S).
* primitive pairs of screened lists (a reading beyond the pages, which print
  no such rule): a primitive pair (alpha, beta) of shells a, b is kept when
  its Gaussian-product exponent q = alpha beta / (alpha + beta) |AB|^2 is at
  most 230 (exp(-q) >= 1.3e-100); a shell pair with none keeps its first.
  K_pair of a screened list counts the kept primitive pairs (``prim_pairs_kept``);
  the oracle's integrals themselves always sum over every primitive pair.
"""
from __future__ import annotations

import numpy as np


def pair_class(la, lb):
    la, lb = max(la, lb), min(la, lb)
    return la * (la + 1) // 2 + lb


def class_id(pcb, pck):
    assert pcb >= pck
    return pcb * (pcb + 1) // 2 + pck


def pair_class_ls(pc):
    la = 0
    while (la + 1) * (la + 2) // 2 <= pc:
        la += 1
    return la, pc - la * (la + 1) // 2


def class_ls(cid):
    pcb = 0
    while (pcb + 1) * (pcb + 2) // 2 <= cid:
        pcb += 1
    pck = cid - pcb * (pcb + 1) // 2
    return pair_class_ls(pcb) + pair_class_ls(pck)


def canonical(l, i, j, k, m):
    perm = 0
    if l[i] < l[j]:
        i, j = j, i
        perm |= 1
    if l[k] < l[m]:
        k, m = m, k
        perm |= 2
    if pair_class(l[i], l[j]) < pair_class(l[k], l[m]):
        i, j, k, m = k, m, i, j
        perm |= 4
    return i, j, k, m, perm


def _blocks(cls):
    blocks = []
    start = 0
    for x in range(1, len(cls) + 1):
        if x == len(cls) or cls[x] != cls[start]:
            blocks.append((int(cls[start]), start, x - start))
            start = x
    return blocks


def explicit_plan(l, nprim, quartets):
    """Plan for an explicit quartet list.

    Returns dict(index_map[n,5] = (a, b, c, d, perm) in plan order,
    order[n] = input position of each plan slot, blocks = [(class, start, count)]).
    """
    l = np.asarray(l)
    nprim = np.asarray(nprim)
    q = np.asarray(quartets).reshape(-1, 4)
    n = len(q)
    im = np.zeros((n, 5), dtype=np.int32)
    cls = np.zeros(n, dtype=np.int64)
    kb = np.zeros(n, dtype=np.int64)
    kk = np.zeros(n, dtype=np.int64)
    for x in range(n):
        a, b, c, d, perm = canonical(l, *[int(v) for v in q[x]])
        im[x] = (a, b, c, d, perm)
        cls[x] = class_id(pair_class(l[a], l[b]), pair_class(l[c], l[d]))
        kb[x] = nprim[a] * nprim[b]
        kk[x] = nprim[c] * nprim[d]
    order = np.lexsort((np.arange(n), kk, kb, cls))
    return {"index_map": im[order], "order": order.astype(np.int64), "blocks": _blocks(cls[order]),
            "class": cls[order]}


PRIM_QMAX = 230.0


def prim_pairs_kept(centers, prim_off, exps, A, B):
    """Kept primitive-pair counts of shell pairs (A[n], B[n]) (see the module
    docstring): q is formed as ((alpha beta) / (alpha + beta)) AB2 with
    AB2 = (dx dx + dy dy) + dz dz, every step a correctly rounded fp64
    operation, so the decision at the threshold is reproducible."""
    centers = np.asarray(centers, dtype=np.float64).reshape(-1, 3)
    prim_off = np.asarray(prim_off, dtype=np.int64)
    exps = np.asarray(exps, dtype=np.float64)
    A = np.asarray(A, dtype=np.int64)
    B = np.asarray(B, dtype=np.int64)
    out = np.zeros(len(A), dtype=np.int64)
    K = prim_off[1:] - prim_off[:-1]
    kmax = int(K.max()) if len(K) else 1
    # exponents padded per shell; padding never counts
    E = np.full((len(K), kmax), np.nan)
    for s_ in range(len(K)):
        E[s_, :K[s_]] = exps[prim_off[s_]:prim_off[s_ + 1]]
    step = 65536
    for c in range(0, len(A), step):
        a, b = A[c:c + step], B[c:c + step]
        d = centers[a] - centers[b]
        ab2 = (d[:, 0] * d[:, 0] + d[:, 1] * d[:, 1]) + d[:, 2] * d[:, 2]
        al = E[a][:, :, None]
        be = E[b][:, None, :]
        with np.errstate(invalid="ignore"):
            q = (al * be) / (al + be) * ab2[:, None, None]
            n = (q <= PRIM_QMAX).sum(axis=(1, 2))
        out[c:c + step] = np.maximum(n, 1)
    return out


def pair_table(l, nprim, S, shells=None):
    """Pairs i >= j with orientation, bucket and in-bucket rank.  K_pair is the
    primitive-pair count nprim[a] nprim[b], or with ``shells`` (centers,
    prim_off, exps) the kept count of a screened list."""
    l = np.asarray(l)
    nprim = np.asarray(nprim)
    ns = len(l)
    pairs = []
    for i in range(ns):
        for j in range(i + 1):
            a, b = (i, j) if l[i] >= l[j] else (j, i)
            pairs.append((i, j, a, b, pair_class(l[a], l[b]), int(nprim[a] * nprim[b])))
    P = np.array(pairs, dtype=np.int64).reshape(-1, 6)
    if shells is not None and len(P):
        P[:, 5] = prim_pairs_kept(shells.centers, shells.prim_off, shells.exps, P[:, 2], P[:, 3])
    S = np.asarray(S, dtype=np.float64)
    npair = len(P)
    pidx = np.arange(npair)
    # bucket order (pc, K); inside a bucket S descending, ties by pair index
    order = np.lexsort((pidx, -S, P[:, 5], P[:, 4]))
    bkeys = P[order][:, 4:6]
    bucket = np.zeros(npair, dtype=np.int64)
    rank = np.zeros(npair, dtype=np.int64)
    bid = -1
    prev = None
    r = 0
    for pos, p in enumerate(order):
        key = (int(bkeys[pos, 0]), int(bkeys[pos, 1]))
        if key != prev:
            bid += 1
            prev = key
            r = 0
        bucket[p] = bid
        rank[p] = r
        r += 1
    return {"pairs": P, "bucket": bucket, "rank": rank, "order": order}


def screened_plan(l, nprim, S, tau, shells=None):
    """All unique quartets that pass fl(S_p S_q) >= fl(tau^2), in plan order.

    S is indexed by pair index i(i+1)/2 + j.  Returns dict(index_map[n,5],
    pair_bra[n], pair_ket[n], blocks, bucket, rank).  The perm bits are taken
    relative to the natural unique form (i >= j, k >= l, pair(ij) >= pair(kl)).
    """
    pt = pair_table(l, nprim, S, shells)
    P, bucket, rank = pt["pairs"], pt["bucket"], pt["rank"]
    S = np.asarray(S, dtype=np.float64)
    npair = len(P)
    t2 = np.float64(tau) * np.float64(tau)
    rows = []
    for p in range(npair):
        # every q with q <= p: the unordered pair {p, q} once
        qs = np.arange(p + 1)
        keep = (S[p] * S[qs]) >= t2
        qs = qs[keep]
        if len(qs) == 0:
            continue
        bp, bq = bucket[p], bucket[qs]
        p_is_bra = (bp > bq) | ((bp == bq) & (rank[p] <= rank[qs]))
        bra = np.where(p_is_bra, p, qs)
        ket = np.where(p_is_bra, qs, p)
        rows.append(np.stack([bra, ket], axis=1))
    if rows:
        BK = np.concatenate(rows)
    else:
        BK = np.zeros((0, 2), dtype=np.int64)
    bra, ket = BK[:, 0], BK[:, 1]
    pcb, pck = P[bra, 4], P[ket, 4]
    cls = pcb * (pcb + 1) // 2 + pck
    kb, kk = P[bra, 5], P[ket, 5]
    order = np.lexsort((rank[ket], rank[bra], kk, kb, cls))
    bra, ket, cls = bra[order], ket[order], cls[order]
    n = len(bra)
    im = np.zeros((n, 5), dtype=np.int32)
    im[:, 0] = P[bra, 2]
    im[:, 1] = P[bra, 3]
    im[:, 2] = P[ket, 2]
    im[:, 3] = P[ket, 3]
    perm = (P[bra, 2] != P[bra, 0]).astype(np.int32) | ((P[ket, 2] != P[ket, 0]).astype(np.int32) << 1) | \
           ((bra < ket).astype(np.int32) << 2)
    im[:, 4] = perm
    return {"index_map": im, "pair_bra": bra, "pair_ket": ket, "blocks": _blocks(cls), "class": cls,
            "bucket": bucket, "rank": rank}


def screened_counts(l, nprim, S, tau, shells=None):
    """Counts of the screened plan without listing its quartets (for plans too
    large to enumerate).  Same rules as ``screened_plan``.

    For each (bra bucket B, ket bucket Bk <= B) and each bra of rank r in B,
    the kets are the pairs of Bk (of rank >= r when Bk == B) with
    fl(S_bra * S_ket) >= fl(tau^2).  Inside a bucket the ranks follow S
    descending, and fl(S_bra * x) never decreases as x grows, so in rank
    order the surviving kets are a prefix; its length is found by bisection
    on the test itself.  Returns dict(blocks = [(class, start, count)],
    groups = [(class, K_bra, K_ket, B, Bk, start, counts[bra rank])] in plan
    order, pairs, bucket_members[b] = pair indices of bucket b in rank order).
    """
    pt = pair_table(l, nprim, S, shells)
    P, bucket, order = pt["pairs"], pt["bucket"], pt["order"]
    S = np.asarray(S, dtype=np.float64)
    t2 = np.float64(tau) * np.float64(tau)
    nb = int(bucket.max()) + 1 if len(bucket) else 0
    members = [order[np.searchsorted(bucket[order], b, side="left"):np.searchsorted(bucket[order], b, side="right")]
               for b in range(nb)]
    groups = []
    for B in range(nb):
        for Bk in range(B + 1):
            bra, ket = members[B], members[Bk]
            pcb, pck = int(P[bra[0], 4]), int(P[ket[0], 4])
            groups.append([class_id(pcb, pck), int(P[bra[0], 5]), int(P[ket[0], 5]), B, Bk])
    groups.sort(key=lambda g: (g[0], g[1], g[2]))
    start = 0
    out = []
    for cid, kb, kk, B, Bk in groups:
        sb, sk = S[members[B]], S[members[Bk]]
        lo = np.zeros(len(sb), dtype=np.int64)
        hi = np.full(len(sb), len(sk), dtype=np.int64)
        if B == Bk:
            lo = np.arange(len(sb), dtype=np.int64)  # kets of rank >= the bra's own
        first = lo.copy()
        # bisection: the first rank in [lo, hi) where the test fails
        while True:
            act = lo < hi
            if not act.any():
                break
            mid = (lo + hi) // 2
            ok = np.zeros(len(sb), dtype=bool)
            ok[act] = (sb[act] * sk[np.minimum(mid[act], len(sk) - 1)]) >= t2
            lo = np.where(act & ok, mid + 1, lo)
            hi = np.where(act & ~ok, mid, hi)
        counts = lo - first
        out.append((cid, kb, kk, B, Bk, start, counts))
        start += int(counts.sum())
    blocks = []
    for g in out:
        n = int(g[6].sum())
        if n == 0:
            continue
        if blocks and blocks[-1][0] == g[0]:
            blocks[-1] = (g[0], blocks[-1][1], blocks[-1][2] + n)
        else:
            blocks.append((g[0], g[5], n))
    return {"blocks": blocks, "groups": out, "pairs": P, "bucket_members": members, "n_quartets": start}


def screened_decode(sc, slots):
    """Index-map rows (a, b, c, d, perm) of the given plan slots of a plan
    described by ``screened_counts``."""
    P, members = sc["pairs"], sc["bucket_members"]
    starts = np.array([g[5] for g in sc["groups"]], dtype=np.int64)
    rows = np.zeros((len(slots), 5), dtype=np.int32)
    for x, s in enumerate(np.asarray(slots, dtype=np.int64)):
        # the last group starting at or before s (empty groups share the next start)
        gi = int(np.searchsorted(starts, s, side="right")) - 1
        cid, kb, kk, B, Bk, st, counts = sc["groups"][gi]
        assert st <= s < st + int(counts.sum())
        off = np.concatenate([[0], np.cumsum(counts)])
        r = int(np.searchsorted(off, s - st, side="right")) - 1
        t = int(s - st - off[r])
        bra = int(members[B][r])
        ket = int(members[Bk][(r if B == Bk else 0) + t])
        perm = int(P[bra, 2] != P[bra, 0]) | (int(P[ket, 2] != P[ket, 0]) << 1) | (int(bra < ket) << 2)
        rows[x] = (P[bra, 2], P[bra, 3], P[ket, 2], P[ket, 3], perm)
    return rows
