"""Plant plausible mistakes in copies of the oracle (CPU only) and require the pins
to reject every one: a pin that no mistake can fail would pin nothing."""

import math

import numpy as np
import pytest

import oracle
from pins import pins_attention, pins_const_max, pins_dcp_active, pins_merge, pins_segmented, pins_sink_robust


def _attn_factory(scale_pow=1, use_max=True, lse_log=np.log, normalise=True, honour_mask=True,
                  lse_adds_max=True, swap_qk_in_pv=False):
    def attn(q, k, v, scale, allowed=None):
        q = np.asarray(q, float); k = np.asarray(k, float); v = np.asarray(v, float)
        Sq, Sk = q.shape[0], k.shape[0]
        o = np.zeros((Sq, v.shape[1])); lse = np.full(Sq, -np.inf)
        if Sk == 0 or Sq == 0:
            return o, lse
        s = (scale ** scale_pow) * (q @ k.T)
        if allowed is not None and honour_mask:
            s = np.where(allowed, s, -np.inf)
        with np.errstate(all="ignore"):
            m = s.max(axis=1) if use_max else np.zeros(Sq)
            m = np.where(np.isfinite(m), m, 0.0)
            e = np.exp(s - m[:, None])
            z = e.sum(axis=1)
            live = z > 0
            lse = np.where(live, (m if lse_adds_max else 0.0) + lse_log(np.where(live, z, 1.0)), -np.inf)
            p = e / np.where(live, z, 1.0)[:, None] if normalise else e
            if swap_qk_in_pv:
                p = p[:, ::-1]
            o = np.where(live[:, None], p @ v, 0.0)
        return o, lse
    return attn


ATTN_MUTANTS = {
    "scale_dropped": _attn_factory(scale_pow=0),
    "scale_squared": _attn_factory(scale_pow=2),
    "no_max_subtraction": _attn_factory(use_max=False),
    "lse_log10": _attn_factory(lse_log=np.log10),
    "unnormalised_output": _attn_factory(normalise=False),
    "mask_ignored": _attn_factory(honour_mask=False),
    "lse_missing_max": _attn_factory(lse_adds_max=False),
    "value_rows_reversed": _attn_factory(swap_qk_in_pv=True),
}


@pytest.mark.parametrize("name", sorted(ATTN_MUTANTS))
def test_attention_mutant_caught(name):
    assert pins_attention(ATTN_MUTANTS[name]), f"{name} passed every attention pin"


def _merge_factory(kind):
    def merge(o_parts, lse_parts):
        L = np.stack([np.asarray(x, float) for x in lse_parts]); O = np.stack([np.asarray(x, float) for x in o_parts])
        with np.errstate(all="ignore"):
            M = L.max(axis=0)
            live = np.isfinite(M)
            Ms = np.where(live, M, 0.0)
            if kind == "no_max":
                g = np.log(np.exp(L).sum(axis=0))
            elif kind == "global_is_max":
                g = M
            else:
                g = np.where(live, Ms + np.log(np.exp(L - Ms).sum(axis=0)), -np.inf)
            gs = np.where(np.isfinite(g), g, 0.0)
            if kind == "inverted_weight":
                w = np.where(np.isfinite(L), np.exp(gs - L), 0.0)
            elif kind == "plain_mean":
                w = np.where(np.isfinite(L), 1.0 / L.shape[0], 0.0)
            else:
                w = np.where(np.isfinite(L), np.exp(L - gs), 0.0)
            out = (w[..., None] * O).sum(axis=0)
        return out, g
    return merge


@pytest.mark.parametrize("kind", ["no_max", "global_is_max", "inverted_weight", "plain_mean"])
def test_merge_mutant_caught(kind):
    assert pins_merge(oracle.attention, _merge_factory(kind)), kind


def _bound_factory(kind):
    def bound(q, k_chunks, scale):
        q = np.asarray(q, float)
        ks = [np.asarray(x, float) for x in k_chunks]
        if kind == "first_chunk_only":
            ks = ks[:1]
        kmax = max(float((x * x).sum(axis=1).max()) for x in ks if len(x))
        qn2 = (q * q).sum(axis=1)
        if kind == "no_sqrt":
            return scale * qn2 * kmax, kmax
        if kind == "no_scale":
            return np.sqrt(qn2 * kmax), kmax
        return scale * np.sqrt(qn2) * math.sqrt(kmax), kmax
    return bound


def _const_max_factory(bound, clamp=1e-37, lse_adds_c=True):
    def cm(q, k_chunks, v_chunks, scale):
        q = np.asarray(q, float)
        c, _ = bound(q, k_chunks, scale)
        Z = np.zeros(q.shape[0]); A = np.zeros((q.shape[0], np.asarray(v_chunks[0]).shape[1]))
        with np.errstate(all="ignore"):
            for kc, vc in zip(k_chunks, v_chunks):
                p = np.exp(scale * (q @ np.asarray(kc, float).T) - c[:, None])
                Z += p.sum(axis=1); A += p @ np.asarray(vc, float)
            Zc = np.maximum(Z, clamp) if clamp else Z
            return A / Zc[:, None], (c if lse_adds_c else 0.0) + np.log(Zc), c
    return cm


CM_MUTANTS = {
    "bound_first_chunk_only": (_bound_factory("first_chunk_only"), {}),
    "bound_no_sqrt": (_bound_factory("no_sqrt"), {}),
    "bound_no_scale": (_bound_factory("no_scale"), {}),
    "no_clamp": (_bound_factory("ok"), {"clamp": 0.0}),
    "clamp_too_high": (_bound_factory("ok"), {"clamp": 1e-30}),
    "lse_missing_c": (_bound_factory("ok"), {"lse_adds_c": False}),
}


@pytest.mark.parametrize("name", sorted(CM_MUTANTS))
def test_const_max_mutant_caught(name):
    bound, kw = CM_MUTANTS[name]
    assert pins_const_max(oracle.attention, _const_max_factory(bound, **kw), bound), name


def test_unmutated_factories_pass():
    """The factories themselves, without a planted mistake, pass: so a caught mutant is
    caught for its mistake, not for a difference in the harness."""
    assert pins_attention(_attn_factory()) == []
    assert pins_merge(oracle.attention, _merge_factory("ok")) == []
    b = _bound_factory("ok")
    assert pins_const_max(oracle.attention, _const_max_factory(b), b) == []


# ---------------------------------------------------------------- DCP decode with the current token

def _active_factory(gate):
    """gate(N, rank, interleave, world) -> whether this rank adds the current token."""
    def partial(q, k, v, ka, va, rank, interleave, world, block_size, scale):
        N = k.shape[0]
        mine = oracle.dcp_shard_of_position(np.arange(N), interleave, world) == rank
        kk, vv = k[mine], v[mine]
        if gate(N, rank, interleave, world):
            kk = np.concatenate([kk, ka[None]]); vv = np.concatenate([vv, va[None]])
        return oracle.decode_full(q, kk, vv, scale)
    return partial


ACTIVE_MUTANTS = {
    "every_rank_adds_it": _active_factory(lambda N, r, I, W: True),
    "no_rank_adds_it": _active_factory(lambda N, r, I, W: False),
    "rank0_adds_it": _active_factory(lambda N, r, I, W: r == 0),
    "owner_of_previous_position": _active_factory(lambda N, r, I, W: ((N - 1) // I) % W == r if N else r == 0),
}


@pytest.mark.parametrize("name", sorted(ACTIVE_MUTANTS))
def test_dcp_active_mutant_caught(name):
    assert any(pins_dcp_active(ACTIVE_MUTANTS[name], W, I) for W, I in ((2, 16), (4, 4), (3, 1))), name


# ---------------------------------------------------------------- DCP prefill (segmented attention)

def _segmented_factory(cur_offset=True, rank_term=True, causal=True, query_offset=True):
    def pos(slots, rank, I, W):
        s = np.asarray(slots)
        return (s // I) * (W * I) + (rank * I if rank_term else 0) + (s % I)

    def partial(q, k_cur, v_cur, k_prior, v_prior, prior_global, rank, I, W, scale):
        k = np.concatenate([k_prior, k_cur]); v = np.concatenate([v_prior, v_cur])
        kpos = np.concatenate([pos(np.arange(k_prior.shape[0]), rank, I, W),
                               (prior_global if cur_offset else 0) + pos(np.arange(k_cur.shape[0]), rank, I, W)])
        qpos = (prior_global if query_offset else 0) + np.arange(q.shape[0])
        allowed = oracle.causal_allowed(qpos, kpos) if causal else None
        Hq, Hkv = q.shape[1], k.shape[1]
        o = np.zeros((Hq, q.shape[0], v.shape[2])); lse = np.zeros((Hq, q.shape[0]))
        for h in range(Hq):
            o[h], lse[h] = oracle.attention(q[:, h], k[:, h * Hkv // Hq], v[:, h * Hkv // Hq], scale, allowed)
        return o, lse
    return partial


SEGMENTED_MUTANTS = {
    "current_slice_without_prior_offset": _segmented_factory(cur_offset=False),
    "positions_without_rank_term": _segmented_factory(rank_term=False),
    "mask_ignored": _segmented_factory(causal=False),
    "queries_without_prior_offset": _segmented_factory(query_offset=False),
}


@pytest.mark.parametrize("name", sorted(SEGMENTED_MUTANTS))
def test_segmented_mutant_caught(name):
    assert any(pins_segmented(SEGMENTED_MUTANTS[name], W, I, pr) for W, I, pr in ((2, 4, 1), (4, 4, 3), (2, 16, 0))), name


def test_segmented_reference_copy_passes():
    """The unmutated copy passes the same pins, so the catches above are the plants'."""
    assert not any(pins_segmented(_segmented_factory(), W, I, pr) for W, I, pr in ((2, 4, 1), (4, 4, 3), (2, 16, 0)))
    assert not any(pins_dcp_active(_active_factory(lambda N, r, I, W: (N // I) % W == r), W, I)
                   for W, I in ((2, 16), (4, 4), (3, 1)))



# ---------------------------------------------------------------- sink-robust const-max

def _robust_factory(bound_over_all=False, drop_sinks=False, double_count=False, theta_on_squares=False):
    def key_sinks(k_chunks, theta, max_sinks):
        k_chunks = [np.asarray(x, float) for x in k_chunks]
        norms = [(kc * kc).sum(axis=1) for kc in k_chunks]
        allv = np.concatenate(norms)
        if theta <= 0 or allv.size == 0:
            return [np.zeros(n.shape[0], bool) for n in norms]
        if theta_on_squares:
            masks = [n > theta * allv.mean() for n in norms]
        else:
            masks = [np.sqrt(n) > theta * np.sqrt(allv).mean() for n in norms]
        if sum(int(m.sum()) for m in masks) > max_sinks:
            return [np.zeros(n.shape[0], bool) for n in norms]
        return masks

    def robust(q, k_chunks, v_chunks, scale, theta, max_sinks):
        masks = key_sinks(k_chunks, theta, max_sinks)
        kn = [kc if double_count else kc[~m] for kc, m in zip(k_chunks, masks)]
        vn = [vc if double_count else vc[~m] for vc, m in zip(v_chunks, masks)]
        ks = np.concatenate([kc[m] for kc, m in zip(k_chunks, masks)])
        vs = np.concatenate([vc[m] for vc, m in zip(v_chunks, masks)])
        if bound_over_all:
            # the fold over the kept keys, but with the bound taken over every key
            c, _ = oracle.const_max_bound(q, k_chunks, scale)
            Z = sum(np.exp(scale * (q @ np.asarray(x, float).T) - c[:, None]).sum(axis=1) for x in kn if len(x))
            A = sum(np.exp(scale * (q @ np.asarray(x, float).T) - c[:, None]) @ np.asarray(y, float)
                    for x, y in zip(kn, vn) if len(x))
            Zc = np.maximum(Z, oracle.SUM_CLAMP)
            o_n, l_n = A / Zc[:, None], c + np.log(Zc)
        else:
            o_n, l_n, c = oracle.const_max(q, kn, vn, scale)
        if drop_sinks:
            return o_n, l_n, c
        o_s, l_s = oracle.attention(q, ks, vs, scale)
        o, l = oracle.merge_lse([o_n, o_s], [l_n, l_s])
        return o, l, c
    return robust, key_sinks


ROBUST_MUTANTS = {
    "bound_over_every_key": _robust_factory(bound_over_all=True),
    "sinks_not_attended": _robust_factory(drop_sinks=True),
    "sinks_counted_twice": _robust_factory(double_count=True),
    "threshold_on_squared_norms": _robust_factory(theta_on_squares=True),
}


@pytest.mark.parametrize("name", sorted(ROBUST_MUTANTS))
def test_sink_robust_mutant_caught(name):
    assert pins_sink_robust(*ROBUST_MUTANTS[name]), name
