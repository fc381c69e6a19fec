"""Checks that tie the fp64 oracle to facts other than itself.

Every pin takes an oracle callable ``fn(q, k, v, scale, causal, valid_len=None, rows=None)``
returning ``(O, LSE)`` in float64, so the same pins run against the real oracle and against
copies of it with planted mistakes (test_oracle_mutants.py). The pins are:

  * a library routine: torch's float64 CPU ``scaled_dot_product_attention`` (with its own
    grouped-query handling, ``enable_gqa``) and ``torch.logsumexp`` over masked scores;
  * identities: with V the identity matrix the output row is the weight vector, and each weight
    equals exp(score - LSE); weights sum to 1 and are exactly 0 on hidden keys;
  * closed forms: Q = 0 gives the mean of V over the visible keys and LSE = ln |J|; constant V
    rows give that row; causal row 0 gives V[0] and LSE = scale*q0.k0; two keys give a
    logistic mix; the worked examples in tests/golden;
  * invariants: key permutation, causal row = attention over the prefix, valid_len = L equals
    truncation to L, GQA equals repeating each KV head for its group of query heads, per-(b, h)
    slices equal single-head calls, adding a constant to every score shifts only the LSE;
  * special cases: fully masked rows give exactly 0 and -inf; very large scores stay finite;
  * explicit masks (MASK_PINS, for callables that also take keep_mask / add_mask): torch's SDPA
    with boolean and float attn_mask, the identities that tie a mask to no mask, to causal
    masking and to valid_len, and the closed form of an additive log-weight mask;
  * the backward (BWD_PINS, BWD_MASK_PINS, for gradient callables ``fn_bwd(q, k, v, dout, scale,
    causal, valid_len=None, **mask)``): torch's fp64 autograd through SDPA (with causal, padding,
    GQA and explicit masks), central finite differences through the forward oracle, the zero-sum
    and exact-zero identities, GQA = repeated KV heads, and the mask identities (no-op masks,
    causal as a mask, keep = additive -inf, per-row shift invariance).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _normal(rng, shape, std=1.0):
    return rng.standard_normal(shape) * std


def _visible_mask(B, N, causal, valid_len):
    """Boolean [B, N(query), N(key)] visibility built with numpy primitives."""
    vis = np.ones((B, N, N), dtype=bool)
    if causal:
        vis &= np.tril(np.ones((N, N), dtype=bool))[None]
    if valid_len is not None:
        vl = np.clip(np.asarray(valid_len), 0, N)
        vis &= (np.arange(N)[None, None, :] < vl[:, None, None])
    return vis


def _tiny_configs():
    for B, Hq, Hkv in ((1, 1, 1), (2, 2, 2), (2, 4, 2), (1, 4, 1), (2, 3, 3), (1, 6, 2)):
        for N in (1, 2, 5, 9):
            for D in (1, 3, 8):
                for causal in (False, True):
                    for padded in (False, True):
                        yield B, Hq, Hkv, N, D, causal, padded


def pin_library_sdpa(fn):
    """Match torch's fp64 CPU SDPA (O) and torch.logsumexp (LSE) over tiny masked cases."""
    count = 0
    for idx, (B, Hq, Hkv, N, D, causal, padded) in enumerate(_tiny_configs()):
        if idx % 3 and not (padded and causal):
            continue  # keep the sweep small; every combination with both masks is kept
        rng = _rng([7, idx])
        q = _normal(rng, (B, Hq, N, D))
        k = _normal(rng, (B, Hkv, N, D))
        v = _normal(rng, (B, Hkv, N, D))
        scale = float(rng.uniform(0.2, 1.5))
        vl = rng.integers(0, N + 1, size=B).astype(np.int32) if padded else None
        O, L = fn(q, k, v, scale, causal, vl)
        vis = _visible_mask(B, N, causal, vl)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        mask = torch.from_numpy(vis)[:, None]            # [B,1,N,N] broadcast over heads
        ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale,
                                             enable_gqa=(Hq != Hkv)).numpy()
        g = Hq // Hkv
        s = torch.matmul(tq, torch.repeat_interleave(tk, g, dim=1).transpose(-1, -2)) * scale
        s = s.masked_fill(~mask, float("-inf"))
        ref_lse = torch.logsumexp(s, dim=-1).numpy()
        nonempty = np.broadcast_to(vis.any(-1)[:, None, :], (B, Hq, N))
        assert np.all(np.isfinite(O)), "non-finite output"
        np.testing.assert_allclose(O[nonempty], ref[nonempty], rtol=0, atol=1e-12)
        np.testing.assert_allclose(L[nonempty], ref_lse[nonempty], rtol=0, atol=1e-12)
        assert np.all(O[~nonempty] == 0.0)
        assert np.all(np.isneginf(L[~nonempty]))
        count += 1
    assert count > 20


def pin_identity_weights(fn):
    """V = identity: the output row is the weight vector; w_j = exp(s_j - LSE) on visible keys
    and exactly 0 on hidden ones; weights sum to 1."""
    for causal in (False, True):
        for vl in (None, np.array([6, 3], np.int32)):
            B, Hq, Hkv, N = 2, 4, 2, 7
            D = N  # V is N x N so that V[j, :] is the j-th unit vector
            rng = _rng([11, causal, vl is None])
            q = _normal(rng, (B, Hq, N, D))
            k = _normal(rng, (B, Hkv, N, D))
            v = np.broadcast_to(np.eye(N), (B, Hkv, N, N)).copy()
            scale = 0.7
            O, L = fn(q, k, v, scale, causal, vl)
            vis = _visible_mask(B, N, causal, vl)
            g = Hq // Hkv
            for b in range(B):
                for h in range(Hq):
                    s = scale * (q[b, h] @ k[b, h // g].T)        # [N, N] scores
                    for i in range(N):
                        w = O[b, h, i]
                        if not vis[b, i].any():
                            assert np.all(w == 0) and np.isneginf(L[b, h, i])
                            continue
                        assert np.all(w[~vis[b, i]] == 0.0), "weight on a hidden key"
                        assert abs(w.sum() - 1.0) < 1e-12, "weights do not sum to 1"
                        expect = np.exp(s[i, vis[b, i]] - L[b, h, i])
                        np.testing.assert_allclose(w[vis[b, i]], expect, rtol=1e-12, atol=0)


def pin_q_zero(fn):
    """Q = 0: every visible score is 0, so O is the mean of V over J and LSE = ln |J|."""
    B, Hq, Hkv, N, D = 2, 4, 2, 6, 5
    rng = _rng(13)
    k = _normal(rng, (B, Hkv, N, D))
    v = _normal(rng, (B, Hkv, N, D))
    q = np.zeros((B, Hq, N, D))
    for causal in (False, True):
        vl = np.array([4, 6], np.int32)
        O, L = fn(q, k, v, 0.9, causal, vl)
        for b in range(B):
            for h in range(Hq):
                for i in range(N):
                    n = min(vl[b], i + 1) if causal else vl[b]
                    np.testing.assert_allclose(O[b, h, i], v[b, h // 2, :n].mean(0), atol=1e-13)
                    assert abs(L[b, h, i] - math.log(n)) < 1e-13


def pin_constant_v(fn):
    """Every V row of a head equal to c: the output is c on every non-empty row."""
    B, Hq, Hkv, N, D = 1, 2, 1, 8, 4
    rng = _rng(17)
    q = _normal(rng, (B, Hq, N, D), 2.0)
    k = _normal(rng, (B, Hkv, N, D), 2.0)
    c = np.array([0.5, -1.25, 3.0, 7.5])
    v = np.broadcast_to(c, (B, Hkv, N, D)).copy()
    for causal in (False, True):
        O, _ = fn(q, k, v, 1.0, causal, None)
        np.testing.assert_allclose(O, np.broadcast_to(c, O.shape), rtol=1e-14, atol=1e-14)


def pin_causal_first_row(fn):
    """Causal row 0 sees only key 0: O = V[0] and LSE = scale * q0 . k0."""
    B, Hq, Hkv, N, D = 2, 2, 1, 5, 6
    rng = _rng(19)
    q = _normal(rng, (B, Hq, N, D))
    k = _normal(rng, (B, Hkv, N, D))
    v = _normal(rng, (B, Hkv, N, D))
    O, L = fn(q, k, v, 0.4, True, None)
    for b in range(B):
        for h in range(Hq):
            np.testing.assert_allclose(O[b, h, 0], v[b, 0, 0], rtol=0, atol=1e-15)
            assert abs(L[b, h, 0] - 0.4 * float(q[b, h, 0] @ k[b, 0, 0])) < 1e-13


def pin_two_keys(fn):
    """N = 2, no mask: O = sigmoid(s0 - s1) V0 + sigmoid(s1 - s0) V1, LSE = logaddexp(s0, s1)."""
    B, Hq, Hkv, N, D = 1, 3, 3, 2, 4
    rng = _rng(23)
    q = _normal(rng, (B, Hq, N, D))
    k = _normal(rng, (B, Hkv, N, D))
    v = _normal(rng, (B, Hkv, N, D))
    scale = 1.3
    O, L = fn(q, k, v, scale, False, None)
    for h in range(Hq):
        for i in range(N):
            s0 = scale * float(q[0, h, i] @ k[0, h, 0])
            s1 = scale * float(q[0, h, i] @ k[0, h, 1])
            a = 1.0 / (1.0 + math.exp(s1 - s0))
            np.testing.assert_allclose(O[0, h, i], a * v[0, h, 0] + (1 - a) * v[0, h, 1],
                                       rtol=0, atol=1e-14)
            assert abs(L[0, h, i] - np.logaddexp(s0, s1)) < 1e-13


def pin_empty_rows(fn):
    """Rows with no visible key give exactly 0 and -inf; valid_len < 0 behaves as 0."""
    B, Hq, Hkv, N, D = 3, 2, 2, 4, 3
    rng = _rng(29)
    q = _normal(rng, (B, Hq, N, D))
    k = _normal(rng, (B, Hkv, N, D))
    v = _normal(rng, (B, Hkv, N, D))
    for causal in (False, True):
        vl = np.array([0, -5, 2], np.int32)
        O, L = fn(q, k, v, 1.0, causal, vl)
        assert np.all(O[:2] == 0.0) and np.all(np.isneginf(L[:2]))
        assert np.all(np.isfinite(O[2])) and np.all(np.isfinite(L[2]))
        assert np.abs(O[2]).max() > 0


def pin_key_permutation(fn):
    """Without masks, permuting key/value rows together changes nothing."""
    B, Hq, Hkv, N, D = 2, 2, 2, 9, 5
    rng = _rng(31)
    q = _normal(rng, (B, Hq, N, D))
    k = _normal(rng, (B, Hkv, N, D))
    v = _normal(rng, (B, Hkv, N, D))
    perm = rng.permutation(N)
    O1, L1 = fn(q, k, v, 0.8, False, None)
    O2, L2 = fn(q, k[:, :, perm], v[:, :, perm], 0.8, False, None)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L1, L2, rtol=0, atol=1e-13)


def pin_causal_prefix(fn):
    """Causal row i equals unmasked attention of that query over keys 0..i."""
    B, Hq, Hkv, N, D = 1, 2, 1, 7, 4
    rng = _rng(37)
    q = _normal(rng, (B, Hq, N, D))
    k = _normal(rng, (B, Hkv, N, D))
    v = _normal(rng, (B, Hkv, N, D))
    O, L = fn(q, k, v, 0.6, True, None)
    for i in range(N):
        qi = np.repeat(q[:, :, i:i + 1], i + 1, axis=2)   # the query, repeated to length i + 1
        Oi, Li = fn(qi, k[:, :, :i + 1], v[:, :, :i + 1], 0.6, False, None)
        np.testing.assert_allclose(O[:, :, i], Oi[:, :, 0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(L[:, :, i], Li[:, :, 0], rtol=0, atol=1e-14)


def pin_valid_len_truncation(fn):
    """valid_len = L equals attention over K[:L], V[:L]; valid_len >= N equals no padding."""
    B, Hq, Hkv, N, D = 1, 2, 2, 8, 3
    rng = _rng(41)
    q = _normal(rng, (B, Hq, N, D))
    k = _normal(rng, (B, Hkv, N, D))
    v = _normal(rng, (B, Hkv, N, D))
    for Lv in (1, 3, 8):
        O, L = fn(q, k, v, 1.1, False, np.array([Lv], np.int32))
        Ot, Lt = fn(q[:, :, :Lv], k[:, :, :Lv], v[:, :, :Lv], 1.1, False, None)
        np.testing.assert_allclose(O[:, :, :Lv], Ot, rtol=0, atol=1e-14)
        np.testing.assert_allclose(L[:, :, :Lv], Lt, rtol=0, atol=1e-14)
    On, Ln = fn(q, k, v, 1.1, True, None)
    for Lv in (N, N + 5):
        Op, Lp = fn(q, k, v, 1.1, True, np.array([Lv], np.int32))
        np.testing.assert_array_equal(On, Op)
        np.testing.assert_array_equal(Ln, Lp)


def pin_gqa_repeat(fn):
    """GQA equals MHA with each KV head repeated for its group of consecutive query heads, and
    differs from the interleaved assignment."""
    B, Hq, Hkv, N, D = 2, 6, 2, 5, 4
    rng = _rng(43)
    q = _normal(rng, (B, Hq, N, D))
    k = _normal(rng, (B, Hkv, N, D))
    v = _normal(rng, (B, Hkv, N, D))
    g = Hq // Hkv
    for causal in (False, True):
        O, L = fn(q, k, v, 0.5, causal, None)
        Or, Lr = fn(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), 0.5, causal, None)
        np.testing.assert_allclose(O, Or, rtol=0, atol=1e-15)
        np.testing.assert_allclose(L, Lr, rtol=0, atol=1e-15)
        Oi, _ = fn(q, np.tile(k, (1, g, 1, 1)), np.tile(v, (1, g, 1, 1)), 0.5, causal, None)
        assert np.abs(O - Oi).max() > 1e-3


def pin_slices(fn):
    """Each (b, hq) slice of a batched call equals a B = 1, single-head call on that slice, so
    batch and head indices are neither swapped nor mixed."""
    B, Hq, Hkv, N, D = 3, 4, 2, 5, 3
    rng = _rng(47)
    q = _normal(rng, (B, Hq, N, D))
    k = _normal(rng, (B, Hkv, N, D))
    v = _normal(rng, (B, Hkv, N, D))
    vl = np.array([5, 2, 4], np.int32)
    for causal in (False, True):
        O, L = fn(q, k, v, 0.9, causal, vl)
        for b in range(B):
            for h in range(Hq):
                kv = h // (Hq // Hkv)
                Os, Ls = fn(q[b:b + 1, h:h + 1], k[b:b + 1, kv:kv + 1], v[b:b + 1, kv:kv + 1],
                            0.9, causal, vl[b:b + 1])
                np.testing.assert_array_equal(O[b, h], Os[0, 0])
                np.testing.assert_array_equal(L[b, h], Ls[0, 0])


def pin_score_shift(fn):
    """Appending a column of ones to Q and a constant c to every key adds scale*c to every score:
    O is unchanged and LSE moves by scale*c, even for shifts far beyond exp's range."""
    B, Hq, Hkv, N, D = 1, 2, 1, 6, 3
    rng = _rng(53)
    q = _normal(rng, (B, Hq, N, D))
    k = _normal(rng, (B, Hkv, N, D))
    v = _normal(rng, (B, Hkv, N, D))
    scale = 0.5
    O, L = fn(q, k, v, scale, True, None)
    for c in (3.0, -4000.0, 4000.0):
        q2 = np.concatenate([q, np.ones((B, Hq, N, 1))], axis=-1)
        k2 = np.concatenate([k, np.full((B, Hkv, N, 1), c)], axis=-1)
        v2 = np.concatenate([v, np.zeros((B, Hkv, N, 1))], axis=-1)
        O2, L2 = fn(q2, k2, v2, scale, True, None)
        np.testing.assert_allclose(O2[..., :D], O, rtol=0, atol=1e-12)
        assert np.all(O2[..., D] == 0.0)
        np.testing.assert_allclose(L2 - scale * c, L, rtol=0, atol=1e-9 * max(1.0, abs(c)))


def pin_large_scores(fn):
    """Q scaled by 30: scores in the hundreds; the output stays finite and matches the library."""
    B, Hq, Hkv, N, D = 1, 2, 2, 9, 8
    rng = _rng(59)
    q = _normal(rng, (B, Hq, N, D)) * 30
    k = _normal(rng, (B, Hkv, N, D))
    v = _normal(rng, (B, Hkv, N, D))
    O, L = fn(q, k, v, 1.0, False, None)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(x) for x in (q, k, v)),
                                         scale=1.0).numpy()
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)


def pin_rows_subset(fn):
    """Asking for a subset of rows returns exactly those rows of the full result."""
    B, Hq, Hkv, N, D = 2, 4, 1, 6, 3
    rng = _rng(61)
    q = _normal(rng, (B, Hq, N, D))
    k = _normal(rng, (B, Hkv, N, D))
    v = _normal(rng, (B, Hkv, N, D))
    vl = np.array([3, 6], np.int32)
    O, L = fn(q, k, v, 0.7, True, vl)
    rows = np.array([0, 5, 7, 23, 30, 47, 13], np.int64)
    Or, Lr = fn(q, k, v, 0.7, True, vl, rows=rows)
    np.testing.assert_array_equal(Or, O.reshape(-1, D)[rows])
    np.testing.assert_array_equal(Lr, L.reshape(-1)[rows])


def pin_golden(fn):
    """Hand-worked examples in tests/golden/closed_form_examples.json; expected values are closed
    forms in e, evaluated here with math."""
    with open(os.path.join(GOLDEN, "closed_form_examples.json")) as f:
        examples = json.load(f)["examples"]
    env = {"e": math.e, "log": math.log, "exp": math.exp, "inf": math.inf}
    for ex in examples:
        q = np.array(ex["q"], np.float64)
        k = np.array(ex["k"], np.float64)
        v = np.array(ex["v"], np.float64)
        vl = None if ex["valid_len"] is None else np.array(ex["valid_len"], np.int32)
        O, L = fn(q, k, v, ex["scale"], ex["causal"], vl)
        exp_o = np.array([[[[eval(t, env) for t in row] for row in head] for head in bat]
                          for bat in ex["expect_o"]], np.float64)
        exp_l = np.array([[[eval(t, env) for t in head] for head in bat]
                          for bat in ex["expect_lse"]], np.float64)
        np.testing.assert_allclose(O, exp_o, rtol=0, atol=1e-14, err_msg=ex["name"])
        fin = np.isfinite(exp_l)
        np.testing.assert_allclose(L[fin], exp_l[fin], rtol=0, atol=1e-14, err_msg=ex["name"])
        assert np.all(L[~fin] == exp_l[~fin]), ex["name"]


# ---- explicit masks: pins take fn(..., keep_mask=None, add_mask=None) as well

def _mask_case(seed, B=2, Hq=4, Hkv=2, N=7, D=5):
    rng = _rng(seed)
    return (rng, _normal(rng, (B, Hq, N, D)), _normal(rng, (B, Hkv, N, D)),
            _normal(rng, (B, Hkv, N, D)))


def pin_mask_library_sdpa(fn):
    """Keep masks and additive masks, per (batch, head) and broadcast, with causal and valid_len:
    match torch's fp64 CPU SDPA (a boolean attn_mask takes part where True, a float attn_mask is
    added to the scaled scores) and torch.logsumexp of the masked scores."""
    count = 0
    for idx in range(12):
        B, Hq, Hkv, N, D = (2, 4, 2, 9, 6) if idx % 2 else (1, 3, 1, 5, 4)
        rng, q, k, v = _mask_case([31, idx], B, Hq, Hkv, N, D)
        causal = bool(idx % 3 == 1)
        vl = rng.integers(0, N + 1, size=B).astype(np.int32) if idx % 4 >= 2 else None
        shape = (B, Hq, N, N) if idx % 5 else (1, 1, N, N)
        scale = float(rng.uniform(0.3, 1.2))
        if idx < 6:
            keep = rng.random(shape) < 0.7
            O, L = fn(q, k, v, scale, causal, vl, keep_mask=keep.astype(np.uint8))
            tmask = torch.from_numpy(np.broadcast_to(keep, (B, Hq, N, N)).copy())
            add = None
        else:
            add = rng.normal(0.0, 2.0, shape)
            add[rng.random(shape) < 0.2] = -np.inf
            O, L = fn(q, k, v, scale, causal, vl, add_mask=add)
            tmask = torch.from_numpy(np.broadcast_to(np.isfinite(add), (B, Hq, N, N)).copy())
        vis = torch.from_numpy(_visible_mask(B, N, causal, vl))[:, None] & tmask
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        g = Hq // Hkv
        tk, tv = torch.repeat_interleave(tk, g, dim=1), torch.repeat_interleave(tv, g, dim=1)
        if add is None:
            ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=vis, scale=scale)
            extra = 0.0
        else:
            fmask = torch.from_numpy(np.broadcast_to(add, (B, Hq, N, N)).copy())
            fmask = fmask.masked_fill(~vis, float("-inf"))
            ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=fmask, scale=scale)
            extra = fmask
        sc = torch.matmul(tq, tk.transpose(-1, -2)) * scale + extra
        sc = sc.masked_fill(~vis, float("-inf"))
        ref_lse = torch.logsumexp(sc, dim=-1).numpy()
        nonempty = vis.any(-1).numpy()
        ref = ref.numpy()
        np.testing.assert_allclose(O[nonempty], ref[nonempty], rtol=0, atol=1e-12)
        np.testing.assert_allclose(L[nonempty], ref_lse[nonempty], rtol=0, atol=1e-12)
        assert np.all(O[~nonempty] == 0.0) and np.all(np.isneginf(L[~nonempty]))
        count += int((~nonempty).sum() > 0)
    assert count >= 2, "no fully masked row was exercised"


def pin_mask_identities(fn):
    """An all-ones keep mask is no mask; a lower-triangular keep mask is causal masking; a
    per-batch length mask is valid_len; an additive 0 is no mask; additive -inf where a keep
    mask is 0 equals that keep mask; an additive constant per row leaves O and shifts LSE."""
    rng, q, k, v = _mask_case([37])
    B, Hq, N = 2, 4, 7
    base_o, base_l = fn(q, k, v, 0.8, False)
    for o, l in (fn(q, k, v, 0.8, False, keep_mask=np.ones((N, N), np.uint8)),
                 fn(q, k, v, 0.8, False, add_mask=np.zeros((B, Hq, N, N)))):
        np.testing.assert_array_equal(o, base_o)
        np.testing.assert_array_equal(l, base_l)
    co, cl = fn(q, k, v, 0.8, True)
    to, tl = fn(q, k, v, 0.8, False, keep_mask=np.tril(np.ones((N, N), np.uint8)))
    np.testing.assert_array_equal(to, co)
    np.testing.assert_array_equal(tl, cl)
    vl = np.array([4, 0], np.int32)
    po, pl = fn(q, k, v, 0.8, True, vl)
    lm = (np.arange(N)[None, None, None, :] < vl[:, None, None, None]).astype(np.uint8)
    mo, ml = fn(q, k, v, 0.8, True, keep_mask=lm)
    np.testing.assert_array_equal(mo, po)
    np.testing.assert_array_equal(ml, pl)
    keep = (rng.random((B, Hq, N, N)) < 0.6).astype(np.uint8)
    ko, kl = fn(q, k, v, 0.8, False, keep_mask=keep)
    ao, al = fn(q, k, v, 0.8, False, add_mask=np.where(keep > 0, 0.0, -np.inf))
    np.testing.assert_array_equal(ao, ko)
    np.testing.assert_array_equal(al, kl)
    shift = rng.normal(0, 3, (B, Hq, N, 1))
    so, sl = fn(q, k, v, 0.8, False, add_mask=np.broadcast_to(shift, (B, Hq, N, N)))
    np.testing.assert_allclose(so, base_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(sl, base_l + shift[..., 0], rtol=0, atol=1e-12)


def pin_mask_log_weights(fn):
    """Additive mask ln w_j with w_j > 0: O = sum_j w_j e^{s_j} V_j / sum_j w_j e^{s_j} and
    LSE = ln sum_j w_j e^{s_j}, evaluated directly for one head."""
    rng, q, k, v = _mask_case([41], B=1, Hq=2, Hkv=1, N=6, D=3)
    w = rng.uniform(0.05, 3.0, (1, 2, 6, 6))
    O, L = fn(q, k, v, 0.6, False, add_mask=np.log(w))
    for h in range(2):
        for i in range(6):
            e = w[0, h, i] * np.exp(0.6 * (k[0, 0] @ q[0, h, i]))
            np.testing.assert_allclose(O[0, h, i], e @ v[0, 0] / e.sum(), rtol=0, atol=1e-12)
            assert abs(L[0, h, i] - math.log(e.sum())) < 1e-12


MASK_PINS = [pin_mask_library_sdpa, pin_mask_identities, pin_mask_log_weights]

# ---- backward: pins take fn_bwd(q, k, v, dout, scale, causal, valid_len=None) -> (dQ, dK, dV)
# and (for the finite-difference pin) the forward callable fn.

def pin_bwd_autograd(fn_bwd, fn=None):
    """torch's fp64 autograd through scaled_dot_product_attention (its own GQA handling) with
    causal and padding masks, on cases where every row sees a key."""
    count = 0
    for idx, (B, Hq, Hkv, N, D, causal, padded) in enumerate(_tiny_configs()):
        if idx % 4:
            continue
        rng = _rng([43, idx])
        q, k, v, do = (_normal(rng, s) for s in ((B, Hq, N, D), (B, Hkv, N, D), (B, Hkv, N, D),
                                                 (B, Hq, N, D)))
        scale = float(rng.uniform(0.2, 1.2))
        vl = rng.integers(1, N + 1, size=B).astype(np.int32) if padded else None
        dq, dk, dv = fn_bwd(q, k, v, do, scale, causal, vl)
        vis = torch.from_numpy(_visible_mask(B, N, causal, vl))[:, None]
        if not bool(vis.any(-1).all()):
            continue
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=vis, scale=scale,
                                           enable_gqa=(Hq != Hkv))
        (o * torch.from_numpy(do)).sum().backward()
        for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-12)
        count += 1
    assert count > 10


def pin_bwd_finite_difference(fn_bwd, fn):
    """Central differences of sum(O * dO), O from the forward callable, on a tiny GQA case
    with causal and padding masks."""
    rng = _rng([47])
    B, Hq, Hkv, N, D = 1, 2, 1, 5, 3
    q, k, v, do = (_normal(rng, s) for s in ((B, Hq, N, D), (B, Hkv, N, D), (B, Hkv, N, D),
                                             (B, Hq, N, D)))
    vl = np.array([4], np.int32)
    dq, dk, dv = fn_bwd(q, k, v, do, 0.8, True, vl)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = float((fn(q, k, v, 0.8, True, vl)[0] * do).sum())
            x[idx] = old - h
            lm = float((fn(q, k, v, 0.8, True, vl)[0] * do).sum())
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=0, atol=1e-7)


def pin_bwd_identities(fn_bwd, fn=None):
    """Softmax rows sum to one, so sum_j dS_ij = 0: the dK of one KV head sums to zero over keys,
    and the dV sums to the dO of its query heads' non-empty rows; hidden keys (past valid_len)
    get dK = dV = 0; rows without a visible key get dQ = 0."""
    rng = _rng([53])
    B, Hq, Hkv, N, D = 2, 4, 2, 9, 6
    q, k, v, do = (_normal(rng, s) for s in ((B, Hq, N, D), (B, Hkv, N, D), (B, Hkv, N, D),
                                             (B, Hq, N, D)))
    vl = np.array([6, 0], np.int32)
    for causal in (False, True):
        dq, dk, dv = fn_bwd(q, k, v, do, 0.6, causal, vl)
        g = Hq // Hkv
        for b in range(B):
            for kv in range(Hkv):
                np.testing.assert_allclose(dk[b, kv].sum(0), 0.0, atol=1e-12)
                expect = np.zeros(D)
                if vl[b] > 0:
                    expect = do[b, kv * g:(kv + 1) * g].sum((0, 1))
                np.testing.assert_allclose(dv[b, kv].sum(0), expect, atol=1e-12)
                assert np.all(dk[b, kv, vl[b]:] == 0) and np.all(dv[b, kv, vl[b]:] == 0)
        assert np.all(dq[1] == 0)     # batch 1 sees no key


def pin_bwd_gqa_repeat(fn_bwd, fn=None):
    """GQA equals MHA on K, V repeated over each group, with dK, dV summed over the group."""
    rng = _rng([59])
    B, Hq, Hkv, N, D = 2, 6, 2, 7, 4
    q, k, v, do = (_normal(rng, s) for s in ((B, Hq, N, D), (B, Hkv, N, D), (B, Hkv, N, D),
                                             (B, Hq, N, D)))
    g = Hq // Hkv
    dq, dk, dv = fn_bwd(q, k, v, do, 0.9, True, np.array([7, 3], np.int32))
    rq, rk, rv = fn_bwd(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), do, 0.9, True,
                        np.array([7, 3], np.int32))
    np.testing.assert_allclose(dq, rq, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk, rk.reshape(B, Hkv, g, N, D).sum(2), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, rv.reshape(B, Hkv, g, N, D).sum(2), rtol=0, atol=1e-13)


def _mask_grad_case(seed, kind, B=2, Hq=4, Hkv=2, N=7, D=5, shape=None):
    """A masked backward case where every row keeps key 0 (no empty rows, which torch's SDPA
    turns into NaN): (rng, q, k, v, dout, mask)."""
    rng = _rng(seed)
    q, k, v, do = (_normal(rng, s) for s in ((B, Hq, N, D), (B, Hkv, N, D), (B, Hkv, N, D),
                                             (B, Hq, N, D)))
    shape = shape or (B, Hq, N, N)
    if kind == "keep":
        m = (rng.random(shape) < 0.6).astype(np.uint8)
        m[..., 0] = 1
    else:
        m = rng.normal(0.0, 2.0, shape)
        m[rng.random(shape) < 0.25] = -np.inf
        m[..., 0] = rng.normal(0.0, 1.0, shape[:-1])
    return rng, q, k, v, do, m


def pin_bwd_mask_autograd(fn_bwd, fn=None):
    """Keep and additive masks (per (batch, head) and broadcast), with causal and valid_len:
    match torch's fp64 autograd through scaled_dot_product_attention given the combined mask as
    its attn_mask (boolean: takes part where True; float: added to the scaled scores)."""
    for idx in range(8):
        kind = "keep" if idx % 2 == 0 else "add"
        B, Hq, Hkv, N, D = (2, 4, 2, 7, 5) if idx < 4 else (1, 3, 1, 9, 3)
        shape = (B, Hq, N, N) if idx % 3 else (1, 1, N, N)
        rng, q, k, v, do, m = _mask_grad_case([61, idx], kind, B, Hq, Hkv, N, D, shape)
        causal = bool(idx % 4 >= 2)
        vl = rng.integers(1, N + 1, size=B).astype(np.int32) if idx in (1, 2, 5, 6) else None
        scale = float(rng.uniform(0.3, 1.2))
        kw = {"keep_mask": m} if kind == "keep" else {"add_mask": m}
        dq, dk, dv = fn_bwd(q, k, v, do, scale, causal, vl, **kw)
        vis = torch.from_numpy(_visible_mask(B, N, causal, vl))[:, None]
        mb = np.broadcast_to(m, (B, Hq, N, N)).copy()
        if kind == "keep":
            tmask = vis & torch.from_numpy(mb.astype(bool))
        else:
            tmask = torch.from_numpy(mb).masked_fill(~vis, float("-inf"))
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=tmask, scale=scale,
                                           enable_gqa=(Hq != Hkv))
        (o * torch.from_numpy(do)).sum().backward()
        for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-12)


def pin_bwd_mask_identities(fn_bwd, fn=None):
    """An all-ones keep mask or an additive 0 gives the unmasked gradients; a lower-triangular
    keep mask gives the causal ones; additive -inf where a keep mask is 0 gives that keep mask's;
    an additive constant per query row changes no gradient (softmax shift invariance)."""
    rng, q, k, v, do, keep = _mask_grad_case([67], "keep")
    B, Hq, N = q.shape[0], q.shape[1], q.shape[2]
    base = fn_bwd(q, k, v, do, 0.7, False)
    causal = fn_bwd(q, k, v, do, 0.7, True)
    vl = np.array([5, 3], np.int32)

    def same(a, b):
        for x, y in zip(a, b):
            np.testing.assert_allclose(x, y, rtol=0, atol=1e-12)

    same(fn_bwd(q, k, v, do, 0.7, False, keep_mask=np.ones((N, N), np.uint8)), base)
    same(fn_bwd(q, k, v, do, 0.7, False, add_mask=np.zeros((B, Hq, N, N))), base)
    same(fn_bwd(q, k, v, do, 0.7, False, keep_mask=np.tril(np.ones((N, N), np.uint8))), causal)
    add = np.where(keep.astype(bool), 0.0, -np.inf)
    same(fn_bwd(q, k, v, do, 0.7, True, vl, add_mask=add),
         fn_bwd(q, k, v, do, 0.7, True, vl, keep_mask=keep))
    shift = rng.normal(0.0, 3.0, (B, Hq, N, 1)) * np.ones((1, 1, 1, N))
    same(fn_bwd(q, k, v, do, 0.7, True, vl, add_mask=shift), fn_bwd(q, k, v, do, 0.7, True, vl))


def pin_bwd_mask_finite_difference(fn_bwd, fn):
    """Central differences of sum(O * dO) through the masked forward callable, with a keep mask
    and with an additive mask, on a tiny causal GQA case."""
    for kind in ("keep", "add"):
        rng, q, k, v, do, m = _mask_grad_case([71, len(kind)], kind, 1, 2, 1, 5, 3)
        kw = {"keep_mask": m} if kind == "keep" else {"add_mask": m}
        dq, dk, dv = fn_bwd(q, k, v, do, 0.8, True, None, **kw)
        h = 1e-6
        for x, g in ((q, dq), (k, dk), (v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                keep = x[idx]
                x[idx] = keep + h
                op = fn(q, k, v, 0.8, True, None, **kw)[0]
                x[idx] = keep - h
                om = fn(q, k, v, 0.8, True, None, **kw)[0]
                x[idx] = keep
                num[idx] = ((op - om) * do).sum() / (2 * h)
            np.testing.assert_allclose(g, num, rtol=0, atol=1e-6)



BWD_PINS = [pin_bwd_autograd, pin_bwd_finite_difference, pin_bwd_identities, pin_bwd_gqa_repeat]
BWD_MASK_PINS = [pin_bwd_mask_autograd, pin_bwd_mask_identities, pin_bwd_mask_finite_difference]

ALL_PINS = [pin_library_sdpa, pin_identity_weights, pin_q_zero, pin_constant_v,
            pin_causal_first_row, pin_two_keys, pin_empty_rows, pin_key_permutation,
            pin_causal_prefix, pin_valid_len_truncation, pin_gqa_repeat, pin_slices,
            pin_score_shift, pin_large_scores, pin_rows_subset, pin_golden]
