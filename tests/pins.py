"""Checks that pin the fp64 oracle to things other than itself.

Each ``pins_*`` function takes the implementation under test as arguments and
returns the names of the checks it fails (empty = pinned). ``test_oracle_pins.py``
runs them on the real oracle; ``test_oracle_mutations.py`` runs them on copies of
the oracle with planted mistakes and requires every mutant to be caught.

The references used here are independent of the oracle's code:
- brute force: pure-Python loops with ``math.exp`` / ``math.fsum``;
- closed forms: one key, zero query, identical keys, constant values, two keys
  (a sigmoid), huge scores (no overflow), empty key sets;
- invariants: shift of all keys, joint permutation of K and V, chunked merge
  equals the unchunked result over contiguous / striped / random partitions with
  empty chunks, merge associativity;
- const-max: Cauchy-Schwarz bound, equality with exact attention when the bound
  overshoots by less than ~85 nats, and the clamp collapse beyond it, including
  the closed form of a single key.
"""

import math

import numpy as np

TOL = 1e-12


def brute_attention(q, k, v, scale, allowed=None):
    """Pure-Python attention with the row log-sum-exp (natural log)."""
    v = np.asarray(v, dtype=np.float64)
    Sq, Sk, Dv = len(q), len(k), v.shape[1]
    out, lses = [], []
    for i in range(Sq):
        s = []
        for j in range(Sk):
            if allowed is not None and not allowed[i][j]:
                continue
            s.append((j, scale * math.fsum(float(a) * float(b) for a, b in zip(q[i], k[j]))))
        if not s:
            out.append([0.0] * Dv)
            lses.append(-math.inf)
            continue
        m = max(x for _, x in s)
        z = math.fsum(math.exp(x - m) for _, x in s)
        lse = m + math.log(z)
        row = [math.fsum(math.exp(x - lse) * float(v[j][d]) for j, x in s) for d in range(Dv)]
        out.append(row)
        lses.append(lse)
    return np.array(out).reshape(Sq, Dv), np.array(lses)


def _close(a, b, tol=TOL):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        return False
    fin = np.isfinite(b)
    if not np.array_equal(np.isfinite(a), fin):
        return False
    if not np.array_equal(a[~fin], b[~fin]):
        return False
    return bool(np.all(np.abs(a[fin] - b[fin]) <= tol * (1.0 + np.abs(b[fin]))))


def pins_attention(attn):
    """attn(q, k, v, scale, allowed=None) -> (O, lse)."""
    bad = []
    rng = np.random.default_rng(7)
    # brute force, with masks including a row with no visible key
    for case in range(6):
        Sq, Sk, D, Dv = rng.integers(1, 7), rng.integers(1, 8), rng.integers(1, 6), rng.integers(1, 5)
        q = rng.normal(size=(Sq, D)) * 1.7
        k = rng.normal(size=(Sk, D))
        v = rng.normal(size=(Sk, Dv))
        scale = 0.3 + 0.2 * case
        allowed = None
        if case % 2:
            allowed = rng.random((Sq, Sk)) < 0.6
            allowed[0, :] = False
        o1, l1 = attn(q, k, v, scale, allowed)
        o2, l2 = brute_attention(q, k, v, scale, allowed)
        if not (_close(o1, o2, 1e-12) and _close(l1, l2, 1e-12)):
            bad.append(f"brute_force[{case}]")
    # one key: O = v0, lse = s00
    q = rng.normal(size=(3, 4)); k = rng.normal(size=(1, 4)); v = rng.normal(size=(1, 2))
    o, l = attn(q, k, v, 0.5)
    if not (_close(o, np.repeat(v, 3, 0)) and _close(l, 0.5 * (q @ k[0]))):
        bad.append("one_key")
    # zero query: O = mean(V), lse = log(Sk)
    k = rng.normal(size=(5, 4)); v = rng.normal(size=(5, 3))
    o, l = attn(np.zeros((2, 4)), k, v, 0.9)
    if not (_close(o, np.repeat(v.mean(0, keepdims=True), 2, 0)) and _close(l, np.full(2, math.log(5)))):
        bad.append("zero_query")
    # identical keys: O = mean(V), lse = s + log(Sk)
    q = rng.normal(size=(2, 4)); k1 = rng.normal(size=(1, 4))
    o, l = attn(q, np.repeat(k1, 6, 0), v[:1].repeat(6, 0) + np.arange(6)[:, None], 0.7)
    want_o = v[:1] + np.arange(6).mean()
    if not (_close(o, np.repeat(want_o, 2, 0)) and _close(l, 0.7 * (q @ k1[0]) + math.log(6))):
        bad.append("identical_keys")
    # constant values: O = that vector
    q = rng.normal(size=(3, 4)); k = rng.normal(size=(7, 4)); cv = rng.normal(size=(1, 5))
    o, _ = attn(q, k, np.repeat(cv, 7, 0), 1.1)
    if not _close(o, np.repeat(cv, 3, 0)):
        bad.append("constant_values")
    # two keys: sigmoid weights
    q = np.array([[1.0, -2.0]]); k = np.array([[0.5, 0.25], [-1.0, 3.0]]); v = np.array([[2.0], [-4.0]])
    s0, s1 = 0.8 * (0.5 - 0.5), 0.8 * (-1.0 - 6.0)
    sig = 1.0 / (1.0 + math.exp(-(s0 - s1)))
    o, l = attn(q, k, v, 0.8)
    if not (_close(o, [[sig * 2.0 + (1 - sig) * -4.0]]) and _close(l, [math.log(math.exp(s0) + math.exp(s1))])):
        bad.append("two_keys")
    # huge scores: no overflow (the max must come off before exp)
    q = np.array([[40.0, 0.0]]); k = np.array([[40.0, 0.0], [39.5, 0.0]]); v = np.array([[1.0], [3.0]])
    o, l = attn(q, k, v, 1.0)
    s0, s1 = 1600.0, 1580.0
    w1 = 1.0 / (1.0 + math.exp(s0 - s1))
    if not (_close(o, [[1.0 * (1 - w1) + 3.0 * w1]]) and _close(l, [s0 + math.log1p(math.exp(s1 - s0))])):
        bad.append("huge_scores")
    # empty key set
    o, l = attn(rng.normal(size=(2, 3)), np.zeros((0, 3)), np.zeros((0, 2)), 1.0)
    if not (np.all(o == 0) and np.all(l == -np.inf) and o.shape == (2, 2)):
        bad.append("empty_keys")
    # shift invariance: k_j -> k_j + u shifts lse by scale*q.u, O unchanged
    q = rng.normal(size=(4, 6)); k = rng.normal(size=(9, 6)); v = rng.normal(size=(9, 3)); u = rng.normal(size=6)
    o1, l1 = attn(q, k, v, 0.4)
    o2, l2 = attn(q, k + u, v, 0.4)
    if not (_close(o1, o2, 1e-11) and _close(l2 - l1, 0.4 * (q @ u), 1e-11)):
        bad.append("shift_invariance")
    # joint permutation of K and V
    perm = rng.permutation(9)
    o3, l3 = attn(q, k[perm], v[perm], 0.4)
    if not (_close(o1, o3, 1e-12) and _close(l1, l3, 1e-12)):
        bad.append("permutation")
    return bad


def pins_merge(attn, merge):
    """merge(o_list, lse_list) -> (O, lse); attn as in ``pins_attention``."""
    bad = []
    rng = np.random.default_rng(11)
    # two partials with known weights: lse log1 and log3 -> 1/4, 3/4
    o, l = merge([np.array([[4.0, 0.0]]), np.array([[0.0, 8.0]])], [np.array([0.0]), np.array([math.log(3.0)])])
    if not (_close(o, [[1.0, 6.0]]) and _close(l, [math.log(4.0)])):
        bad.append("two_partials")
    # all partials empty
    o, l = merge([np.ones((2, 3)), np.ones((2, 3))], [np.full(2, -np.inf), np.full(2, -np.inf)])
    if not (np.all(o == 0) and np.all(l == -np.inf)):
        bad.append("all_empty")
    # one partial empty: result is the other one
    o, l = merge([np.full((1, 2), 5.0), np.array([[1.0, 2.0]])], [np.array([-np.inf]), np.array([2.5])])
    if not (_close(o, [[1.0, 2.0]]) and _close(l, [2.5])):
        bad.append("one_empty")
    # huge lse values do not overflow
    o, l = merge([np.array([[1.0]]), np.array([[3.0]])], [np.array([1000.0]), np.array([1000.0])])
    if not (_close(o, [[2.0]]) and _close(l, [1000.0 + math.log(2.0)])):
        bad.append("huge_lse")
    # chunked merge equals unchunked: contiguous, striped, random, with empty chunks
    Sq, Sk, D = 5, 24, 4
    q = rng.normal(size=(Sq, D)) * 1.5; k = rng.normal(size=(Sk, D)); v = rng.normal(size=(Sk, 3))
    full_o, full_l = attn(q, k, v, 0.6)
    parts = {
        "contiguous4": [np.arange(6 * r, 6 * r + 6) for r in range(4)],
        "striped3": [np.arange(r, Sk, 3) for r in range(3)],
        "random5_with_empty": np.array_split(rng.permutation(Sk), 4) + [np.array([], dtype=int)],
        "single": [np.arange(Sk)],
    }
    for name, idx in parts.items():
        os_, ls_ = zip(*[attn(q, k[i], v[i], 0.6) for i in idx])
        o, l = merge(list(os_), list(ls_))
        if not (_close(o, full_o, 1e-11) and _close(l, full_l, 1e-11)):
            bad.append(f"chunked_{name}")
    # causal mask split across chunks (fully masked rows inside chunks)
    pos_q = np.array([0, 5, 11, 17, 23]); pos_k = np.arange(Sk)
    allowed = pos_q[:, None] >= pos_k[None, :]
    full_o, full_l = attn(q, k, v, 0.6, allowed)
    os_, ls_ = zip(*[attn(q, k[6 * r:6 * r + 6], v[6 * r:6 * r + 6], 0.6, allowed[:, 6 * r:6 * r + 6]) for r in range(4)])
    o, l = merge(list(os_), list(ls_))
    if not (_close(o, full_o, 1e-11) and _close(l, full_l, 1e-11)):
        bad.append("chunked_causal")
    # associativity
    a, b, c = (attn(q, k[i], v[i], 0.6) for i in (np.arange(0, 7), np.arange(7, 15), np.arange(15, 24)))
    ab = merge([a[0], b[0]], [a[1], b[1]])
    o1, l1 = merge([ab[0], c[0]], [ab[1], c[1]])
    o2, l2 = merge([a[0], b[0], c[0]], [a[1], b[1], c[1]])
    if not (_close(o1, o2, 1e-12) and _close(l1, l2, 1e-12)):
        bad.append("associativity")
    return bad


def pins_const_max(attn, const_max, bound):
    """const_max(q, k_chunks, v_chunks, scale) -> (O, lse, c);
    bound(q, k_chunks, scale) -> (c, kmax_sq)."""
    bad = []
    rng = np.random.default_rng(13)
    q = rng.normal(size=(6, 8)); ks = [rng.normal(size=(5, 8)) for _ in range(3)]
    vs = [rng.normal(size=(5, 4)) for _ in range(3)]
    k_all = np.concatenate(ks); v_all = np.concatenate(vs)
    c, kmax_sq = bound(q, ks, 0.35)
    # the bound by its definition, by brute force
    want_kmax = max(math.fsum(x * x for x in row) for row in k_all)
    want_c = [0.35 * math.sqrt(math.fsum(x * x for x in row)) * math.sqrt(want_kmax) for row in q]
    if not (_close(c, want_c) and _close([kmax_sq], [want_kmax])):
        bad.append("bound_definition")
    # the bound is an upper bound on every score (Cauchy-Schwarz)
    if not np.all(0.35 * (q @ k_all.T) <= c[:, None] + 1e-12):
        bad.append("bound_is_upper")
    # the largest key sits in the last chunk: the max must span all chunks
    ks2 = [x.copy() for x in ks]; ks2[-1][2] *= 5.0
    c2, _ = bound(q, ks2, 0.35)
    if not _close(c2, 0.35 * np.linalg.norm(q, axis=1) * np.linalg.norm(ks2[-1][2])):
        bad.append("bound_spans_chunks")
    # equals exact attention when the overshoot is moderate
    o, l, _ = const_max(q, ks, vs, 0.35)
    eo, el = attn(q, k_all, v_all, 0.35)
    if not (_close(o, eo, 1e-11) and _close(l, el, 1e-11)):
        bad.append("equals_exact")
    # single key with an overshoot of delta nats: sum = exp(-delta); clamp at 1e-37
    for delta, name in ((80.0, "overshoot_80"), (90.0, "overshoot_90")):
        qd = np.array([[1.0, 0.0]])
        k_hit = np.array([[0.0, 0.0]])            # the key the row attends: score 0
        k_far = np.array([[0.0, delta]])          # a loud key the row does not see at all... orthogonal
        vv = np.array([[2.0], [7.0]])
        # scores: 0 and 0; bound c = 1 * |q| * delta = delta -> each term exp(-delta)
        o, l, cc = const_max(qd, [k_hit, k_far], [vv[:1], vv[1:]], 1.0)
        z = 2.0 * math.exp(-delta)
        zc = max(z, 1e-37)
        want_o = (2.0 + 7.0) * math.exp(-delta) / zc
        want_l = delta + math.log(zc)
        if not (_close(cc, [delta]) and _close(o, [[want_o]], 1e-9) and _close(l, [want_l], 1e-9)):
            bad.append(name)
    # at 80 nats it still matches exact attention; at 90 it has collapsed
    o80, l80, _ = const_max(np.array([[1.0, 0.0]]), [np.zeros((1, 2)), np.array([[0.0, 80.0]])],
                            [np.array([[2.0]]), np.array([[7.0]])], 1.0)
    if not (_close(o80, [[4.5]], 1e-9) and _close(l80, [math.log(2.0)], 1e-9)):
        bad.append("no_collapse_at_80")
    o90, _, _ = const_max(np.array([[1.0, 0.0]]), [np.zeros((1, 2)), np.array([[0.0, 90.0]])],
                          [np.array([[2.0]]), np.array([[7.0]])], 1.0)
    if abs(float(o90[0, 0]) - 4.5) < 1.0:
        bad.append("collapse_at_90")
    return bad


def pins_dcp_active(partial_active, world, interleave):
    """DCP decode with the current token (DCP page, dcp_active_mask): the W partials merge
    to full attention over the N prior tokens plus the current one, and each partial equals
    brute force over the keys listed from the slot mapping (the owner taken from the
    position, not from the vblock rule). Returns the failures."""
    import oracle
    bad = []
    rng = np.random.default_rng(100 * world + interleave)
    Hq, Hkv, D, bs = 4, 2, 3, 16
    for N in (0, 1, 15, 16, 17, 40, 63, 64, 65, 100):
        q = rng.normal(size=(Hq, D)) * 2
        k = rng.normal(size=(N, Hkv, D)); v = rng.normal(size=(N, Hkv, 2))
        ka = rng.normal(size=(Hkv, D)) * 2; va = rng.normal(size=(Hkv, 2))
        parts = [partial_active(q, k, v, ka, va, r, interleave, world, bs, 0.5) for r in range(world)]
        o, l = oracle.merge_lse([p[0] for p in parts], [p[1] for p in parts])
        fo, fl = oracle.decode_full(q, np.concatenate([k, ka[None]]), np.concatenate([v, va[None]]), 0.5)
        if not (np.allclose(o, fo, atol=TOL) and np.allclose(l, fl, atol=TOL)):
            bad.append(f"merge != full at N={N}")
        for r in range(world):
            keys = [p for p in range(N) if (p // interleave) % world == r]
            kk, vv = k[keys], v[keys]
            if (N // interleave) % world == r:
                kk = np.concatenate([kk, ka[None]]); vv = np.concatenate([vv, va[None]])
            for h in range(Hq):
                bo, bl = brute_attention(q[h:h + 1], kk[:, h // 2], vv[:, h // 2], 0.5)
                if not (np.allclose(parts[r][0][h], bo[0], atol=TOL) and _close(parts[r][1][h], bl[0])):
                    bad.append(f"partial of rank {r} at N={N}, head {h}")
    return bad


def pins_segmented(seg_partial, world, interleave, prior_rounds):
    """DCP prefill (DCP page, segmented attention): every rank's partial over its prior
    slots and its slice of the chunk, causal on global positions, merges to causal
    attention of the chunk's queries over the whole context; one query of one rank by brute
    force. Rank slices are enumerated from the slot mapping. Returns the failures."""
    import oracle
    bad = []
    rng = np.random.default_rng(7 * world + interleave + 100 * prior_rounds)
    Hq, Hkv, D = 4, 2, 3
    rnd = world * interleave
    P = prior_rounds * rnd            # prior tokens: whole interleave rounds, as earlier chunks leave
    S = 2 * rnd                        # chunk length: a multiple of W * I
    q = rng.normal(size=(S, Hq, D)) * 1.5
    k = rng.normal(size=(P + S, Hkv, D)); v = rng.normal(size=(P + S, Hkv, 2))
    parts = []
    for r in range(world):
        prior = [p for p in range(P) if (p // interleave) % world == r]
        cur = [P + j for j in range(S) if (j // interleave) % world == r]
        parts.append(seg_partial(q, k[cur], v[cur], k[prior], v[prior], P, r, interleave, world, 0.7))
    o, l = oracle.merge_lse([p[0] for p in parts], [p[1] for p in parts])
    allowed = oracle.causal_allowed(P + np.arange(S), np.arange(P + S))
    for h in range(Hq):
        fo, fl = brute_attention(q[:, h], k[:, h // 2], v[:, h // 2], 0.7, allowed)
        if not (np.allclose(o[h], fo, atol=TOL) and np.allclose(l[h], fl, atol=TOL)):
            bad.append(f"merge != causal attention, head {h}")
    r = world - 1
    keys = [p for p in range(P + S) if (p // interleave) % world == r and p <= P + S - 2]
    bo, bl = brute_attention(q[S - 2:S - 1, 1], k[keys, 0], v[keys, 0], 0.7)
    if not (np.allclose(parts[r][0][1, S - 2], bo[0], atol=TOL) and _close(parts[r][1][1, S - 2], bl[0])):
        bad.append("one query of the last rank")
    return bad


def pins_sink_robust(robust, key_sinks):
    """robust(q, k_chunks, v_chunks, scale, theta, max_sinks) -> (O, lse, c);
    key_sinks(k_chunks, theta, max_sinks) -> masks. Sinks: keys whose |k| exceeds theta
    times the mean key norm of the ring; the bound then spans the other keys. Returns the
    failures."""
    bad = []
    rng = np.random.default_rng(29)
    D = 8
    q = rng.normal(size=(7, D)) * 3.0
    ks = [rng.normal(size=(6, D)) for _ in range(3)]
    vs = [rng.normal(size=(6, 3)) for _ in range(3)]
    # two keys with norms far above the rest (massive-activation sinks)
    ks[0][4] *= 60.0
    ks[2][1] = -ks[2][1] * 45.0
    k_all = np.concatenate(ks); v_all = np.concatenate(vs)
    masks = key_sinks(ks, 4.0, 32)
    n2 = (k_all * k_all).sum(axis=1)
    want = np.sqrt(n2) > 4.0 * np.sqrt(n2).mean()
    if not np.array_equal(np.concatenate(masks), want) or int(want.sum()) != 2:
        bad.append("sink_selection")
    # equals exact attention (by brute force), where the plain bound collapses every row
    o, l, c = robust(q, ks, vs, 0.5, 4.0, 32)
    bo, bl = brute_attention(q, k_all, v_all, 0.5)
    if not (_close(o, bo, 1e-10) and _close(l, bl, 1e-10)):
        bad.append("equals_exact_with_sinks")
    # the bound spans the non-sink keys only, and still bounds each of their scores
    kmax_n = max(n2[~want])
    if not _close(c, 0.5 * np.linalg.norm(q, axis=1) * math.sqrt(kmax_n)):
        bad.append("bound_without_sinks")
    if not np.all(0.5 * (q @ k_all[~want].T) <= c[:, None] + 1e-12):
        bad.append("bound_is_upper_for_the_rest")
    # too many candidates: no exclusion (the plain bound), still exact here (no collapse)
    masks1 = key_sinks(ks, 4.0, 1)
    if any(m.any() for m in masks1):
        bad.append("cap_disables_exclusion")
    # without sinks nothing is excluded and the result is exact attention
    ks3 = [rng.normal(size=(6, D)) for _ in range(3)]
    o3, l3, _ = robust(q, ks3, vs, 0.5, 4.0, 32)
    bo3, bl3 = brute_attention(q, np.concatenate(ks3), v_all, 0.5)
    if any(m.any() for m in key_sinks(ks3, 4.0, 32)) or not (_close(o3, bo3, 1e-10) and _close(l3, bl3, 1e-10)):
        bad.append("no_sinks_plain")
    # the reference is the mean of the norms: a key 4x louder than thirty unit keys stays
    # below 4 x mean norm (4.39), though its square is far above 4 x the mean square
    unit = np.eye(D)[np.arange(30) % D]
    loud = np.zeros((1, D)); loud[0, 0] = 4.0
    if any(m.any() for m in key_sinks([unit, loud], 4.0, 32)):
        bad.append("reference_is_mean_norm")
    loud[0, 0] = 5.0   # now above 4 x mean norm (4.52)
    if not key_sinks([unit, loud], 4.0, 32)[1].all():
        bad.append("reference_is_mean_norm_above")
    # theta <= 0 disables exclusion
    if any(m.any() for m in key_sinks(ks, 0.0, 32)):
        bad.append("theta_off")
    # an empty chunk and a chunk made only of sinks
    ks4 = [ks[0], np.zeros((0, D)), ks[1], 80.0 * rng.normal(size=(1, D))]
    vs4 = [vs[0], np.zeros((0, 3)), vs[1], rng.normal(size=(1, 3))]
    if sum(int(m.sum()) for m in key_sinks(ks4, 4.0, 32)) != 2:
        bad.append("sink_only_chunk_selection")
    o4, l4, _ = robust(q, ks4, vs4, 0.5, 4.0, 32)
    bo4, bl4 = brute_attention(q, np.concatenate(ks4), np.concatenate(vs4), 0.5)
    if not (_close(o4, bo4, 1e-10) and _close(l4, bl4, 1e-10)):
        bad.append("empty_and_sink_only_chunks")
    return bad
