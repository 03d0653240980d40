"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each ``pin_*`` takes the oracle module and raises AssertionError when the
oracle disagrees with a value printed on the pages (fixtures under
tests/golden/), a closed form, a library routine (torch / scipy), an
invariant, or brute force on tiny inputs.  tests/test_oracle_pins.py runs
them on the real oracle; tests/test_oracle_mutations.py plants mistakes in
the oracle and checks that some pin catches each one.
"""

from __future__ import annotations

import json
import math
import os
from itertools import product

import numpy as np
import scipy.special
import scipy.stats
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _torch_ffn(X, W1, W3, W2):
    """Library reference: torch fp64 SwiGLU FFN."""
    X = torch.as_tensor(np.asarray(X, dtype=np.float64))
    W1 = torch.as_tensor(np.asarray(W1, dtype=np.float64))
    W3 = torch.as_tensor(np.asarray(W3, dtype=np.float64))
    W2 = torch.as_tensor(np.asarray(W2, dtype=np.float64))
    h = torch.nn.functional.silu(X @ W1) * (X @ W3)
    return (h @ W2).numpy()


def _experts(n, d, F, seed):
    r = _rng(seed)
    return [(r.standard_normal((d, F)) / math.sqrt(d),
             r.standard_normal((d, F)) / math.sqrt(d),
             r.standard_normal((F, d)) / math.sqrt(F)) for _ in range(n)]


# ---------------------------------------------------------------- capacity
def pin_capacity_worked_example(O):
    g = golden("capacity_worked_example.json")
    assert O.capacity(g["tokens"], g["top_k"], g["experts"],
                      g["capacity_factor"]) == g["capacity"]


def pin_capacity_rounding(O):
    # Exact decimal reading: 100 tokens x 2 x 1.1 / 2 = 110 exactly (a binary
    # double product would land just above 110 and round up to 111).
    assert O.capacity(100, 2, 2, 1.1) == 110
    # Non-integer value rounds up (the reading for the page's "about").
    assert O.capacity(10, 1, 4, 1.0) == 3
    assert O.capacity(1, 1, 8, 1.0) == 1
    # The recommended range brackets the worked example's factor.
    g = golden("recommended_capacity_factor.json")
    lo = O.capacity(2048, 2, 8, g["low"])
    hi = O.capacity(2048, 2, 8, g["high"])
    assert (lo, hi) == (640, 768)
    # No limit: an expert can take every token once.
    for T in (0, 1, 7, 2048):
        assert O.capacity(T, 2, 8, 0.0) == T
        assert O.capacity(T, 2, 8, -1.0) == T


# ---------------------------------------------------------------- router
def pin_router_one_hot(O):
    # With d == E and one-hot token vectors, token t = e_c must score exactly
    # row c of W_gate plus the bias; a transposed W_gate or a wrong bias sign
    # breaks this.
    r = _rng(1)
    E = 5
    Wg = r.standard_normal((E, E))
    b = r.standard_normal(E)
    x = np.eye(E)
    got = O.router_logits(x, Wg, b)
    assert np.array_equal(got, Wg + b[None, :])
    got0 = O.router_logits(x, Wg, None)
    assert np.array_equal(got0, Wg)


# ---------------------------------------------------------------- top-k
def _check_order(row, sel):
    vals = [row[i] for i in sel]
    for j in range(len(sel) - 1):
        assert vals[j] >= vals[j + 1]
        if vals[j] == vals[j + 1]:
            assert sel[j] < sel[j + 1]


def pin_topk_bruteforce(O):
    r = _rng(2)
    cases = []
    for E in (1, 2, 3, 5, 8):
        for _ in range(40):
            row = r.standard_normal(E)
            # inject exact ties, signed zeros and duplicates
            if E > 1 and r.random() < 0.5:
                i, j = r.choice(E, 2, replace=False)
                row[j] = row[i]
            if r.random() < 0.3:
                row[r.integers(E)] = 0.0
                row[r.integers(E)] = -0.0
            if r.random() < 0.2:
                row[:] = np.round(row)
            cases.append(row)
    cases.append(np.zeros(8))
    cases.append(np.array([-0.0, 0.0, -0.0, 0.0]))
    for row in cases:
        E = len(row)
        for k in range(1, E + 1):
            sel, _ = O.topk_select(row[None, :], k)
            sel = [int(v) for v in sel[0]]
            assert tuple(sorted(sel)) == O.brute_topk_set(row, k), (row, k)
            _check_order(row, sel)


def pin_topk_signed_zero(O):
    sel, margin = O.topk_select(np.array([[-0.0, 0.0, -1.0]]), 1)
    assert sel[0, 0] == 0 and margin[0] == 0.0
    sel, _ = O.topk_select(np.array([[0.0, -0.0, -1.0]]), 2)
    assert list(sel[0]) == [0, 1]
    sel, _ = O.topk_select(np.array([[-1.0, -0.0, 0.0]]), 2)
    assert list(sel[0]) == [1, 2]


def pin_topk_margin(O):
    row = np.array([[3.0, 1.0, 2.5, 0.5]])
    _, m = O.topk_select(row, 2)       # sorted 3, 2.5, 1 -> gaps .5, 1.5
    assert m[0] == 0.5
    _, m = O.topk_select(row, 1)       # 3, 2.5
    assert m[0] == 0.5
    _, m = O.topk_select(np.array([[4.0, 1.0, 3.9]]), 3)  # 4, 3.9, 1
    assert abs(m[0] - 0.1) < 1e-12


# ---------------------------------------------------------------- gates
def pin_gates_topk_then_softmax(O):
    r = _rng(3)
    L = r.standard_normal((50, 8)) * 3
    sel, _ = O.topk_select(L, 2)
    w = O.gate_weights(L, sel, O.TOPK_THEN_SOFTMAX, True)
    for t in range(50):
        l0, l1 = L[t, sel[t, 0]], L[t, sel[t, 1]]
        # two-way softmax is the logistic function of the logit gap
        assert abs(w[t, 0] - 1.0 / (1.0 + math.exp(l1 - l0))) < 1e-15
        assert abs(w[t].sum() - 1.0) < 1e-15
    for k in (1, 3, 8):
        sel, _ = O.topk_select(L, k)
        w = O.gate_weights(L, sel, O.TOPK_THEN_SOFTMAX, True)
        ref = scipy.special.softmax(np.take_along_axis(L, sel, 1), axis=1)
        assert np.allclose(w, ref, rtol=0, atol=1e-15)


def pin_gates_softmax_then_topk(O):
    r = _rng(4)
    L = r.standard_normal((40, 16)) * 2
    sel, _ = O.topk_select(L, 6)
    p = scipy.special.softmax(L, axis=1)
    w = O.gate_weights(L, sel, O.SOFTMAX_THEN_TOPK, False)
    assert np.allclose(w, np.take_along_axis(p, sel, 1), rtol=0, atol=1e-15)
    assert np.all(w.sum(1) <= 1 + 1e-15)
    wn = O.gate_weights(L, sel, O.SOFTMAX_THEN_TOPK, True)
    assert np.allclose(wn.sum(1), 1.0, rtol=0, atol=1e-15)
    assert np.allclose(O.softmax_all(L), p, rtol=0, atol=1e-15)


# ---------------------------------------------------------------- dispatch
def pin_dispatch_stable_sort(O):
    r = _rng(5)
    for (T, E, k, C) in [(37, 4, 2, 9), (64, 8, 2, 16), (50, 5, 3, 1000),
                         (29, 3, 1, 4), (40, 8, 8, 40), (33, 6, 2, 1)]:
        L = r.standard_normal((T, E))
        L[:, 0] += 1.0   # skew so some experts overflow
        sel, _ = O.topk_select(L, k)
        D = O.dispatch(sel, E, C)
        flat = sel.reshape(-1)
        order = sorted(range(T * k), key=lambda a: int(flat[a]))  # stable
        ref_perm = []
        for e in range(E):
            mine = [a for a in order if flat[a] == e]
            ref_perm += mine[:C]
        assert list(D["perm"]) == ref_perm
        cnt = np.bincount(flat, minlength=E)
        assert np.array_equal(D["counts"], cnt)
        assert np.array_equal(D["kept"], np.minimum(cnt, C))
        assert int(D["kept"].sum()) == T * k - D["dropped"]
        assert np.all(D["kept"] <= C)
        for e in range(E):
            if cnt[e] <= C:
                assert D["kept"][e] == cnt[e]
        assert D["offsets"][0] == 0
        assert np.array_equal(np.diff(D["offsets"]), D["kept"])
        for a in range(T * k):
            s = D["slot"][a]
            if s >= 0:
                assert D["perm"][s] == a
        assert int((D["slot"] >= 0).sum()) == len(D["perm"])


def pin_dispatch_hand_example(O):
    # Four tokens, one expert choice each, all on expert 0, two slots:
    # the two earliest tokens keep their slots, the later two are dropped.
    sel = np.array([[0], [0], [0], [0]])
    D = O.dispatch(sel, 2, 2)
    assert list(D["slot"]) == [0, 1, -1, -1]
    assert list(D["perm"]) == [0, 1]
    assert D["dropped"] == 2 and list(D["counts"]) == [4, 0]
    # Two choices per token: expert order inside a token does not change the
    # token-order priority.
    sel = np.array([[1, 0], [0, 1], [1, 2]])
    D = O.dispatch(sel, 3, 1)
    # expert 0: a=1 (t0) kept; a=2 (t1) dropped.  expert 1: a=0 kept,
    # a=3 and a=4 dropped.  expert 2: a=5 kept.
    assert list(D["slot"]) == [1, 0, -1, -1, -1, 2]
    assert list(D["perm"]) == [1, 0, 5]
    assert list(D["offsets"]) == [0, 1, 2, 3]


# ---------------------------------------------------------------- FFN
def pin_ffn_library(O):
    r = _rng(6)
    for (n, d, F) in [(7, 16, 24), (3, 8, 8), (5, 12, 12)]:
        X = r.standard_normal((n, d))
        W1, W3, W2 = _experts(1, d, F, 60 + n)[0]
        got = O.expert_ffn(X, W1, W3, W2)
        assert np.allclose(got, _torch_ffn(X, W1, W3, W2), rtol=1e-13,
                           atol=1e-13)
    u = np.array([-800.0, -30.0, -1.0, 0.0, 2.0, 40.0])
    ref = torch.nn.functional.silu(torch.tensor(u, dtype=torch.float64))
    assert np.allclose(O.silu(u), ref.numpy(), rtol=1e-15, atol=0)


def _shape(O, T, d, F, E, k, S=0, gating=None, renorm=True, cf=0.0,
           overflow=None):
    return O.LayerShape(T=T, d=d, F=F, E=E, k=k, S=S,
                        gating=O.TOPK_THEN_SOFTMAX if gating is None else gating,
                        renormalize=renorm, capacity_factor=cf,
                        overflow=O.OVERFLOW_DROP if overflow is None else overflow)


def pin_dense_equivalence(O):
    # k = E, Mixtral gating, no limit: every expert runs on every token and
    # the layer is the softmax-weighted dense sum; with W_gate = 0 the
    # weights are uniform and it is the plain mean of the experts.
    r = _rng(7)
    T, d, F, E = 12, 16, 20, 4
    x = r.standard_normal((T, d))
    ex = _experts(E, d, F, 70)
    dense = [_torch_ffn(x, *ex[e]) for e in range(E)]
    res = O.forward(x, _shape(O, T, d, F, E, E), lambda e: ex[e],
                    W_gate=np.zeros((d, E)))
    assert np.allclose(res["out"], sum(dense) / E, rtol=1e-12, atol=1e-12)
    Wg = r.standard_normal((d, E))
    res = O.forward(x, _shape(O, T, d, F, E, E), lambda e: ex[e], W_gate=Wg)
    p = scipy.special.softmax(x @ Wg, axis=1)
    ref = sum(p[:, e:e + 1] * dense[e] for e in range(E))
    assert np.allclose(res["out"], ref, rtol=1e-12, atol=1e-12)


def pin_identical_experts(O):
    r = _rng(8)
    T, d, F, E = 10, 8, 12, 6
    x = r.standard_normal((T, d))
    one = _experts(1, d, F, 80)[0]
    Wg = r.standard_normal((d, E))
    ref = _torch_ffn(x, *one)
    res = O.forward(x, _shape(O, T, d, F, E, 2), lambda e: one, W_gate=Wg)
    assert np.allclose(res["out"], ref, rtol=1e-12, atol=1e-12)
    # DeepSeek gating, unrenormalised, plus shared experts: the routed part
    # is (sum of kept probabilities) x FFN.
    sh = _experts(2, d, F, 81)
    experts = lambda e: one if e < E else sh[e - E]  # noqa: E731
    res = O.forward(x, _shape(O, T, d, F, E, 3, S=2,
                              gating=O.SOFTMAX_THEN_TOPK, renorm=False),
                    experts, W_gate=Wg)
    p = scipy.special.softmax(x @ Wg, axis=1)
    top = np.sort(p, axis=1)[:, ::-1][:, :3].sum(1)
    shared = _torch_ffn(x, *sh[0]) + _torch_ffn(x, *sh[1])
    assert np.allclose(res["out"], top[:, None] * ref + shared, rtol=1e-12,
                       atol=1e-12)


def pin_shared_concat(O):
    # S shared experts summed with gate 1 equal one FFN whose hidden layer is
    # the concatenation of theirs.
    r = _rng(9)
    T, d, F, E, S = 9, 8, 6, 4, 2
    x = r.standard_normal((T, d))
    ex = _experts(E + S, d, F, 90)
    Wg = r.standard_normal((d, E))
    with_s = O.forward(x, _shape(O, T, d, F, E, 2, S=S), lambda e: ex[e],
                       W_gate=Wg)["out"]
    without = O.forward(x, _shape(O, T, d, F, E, 2, S=0), lambda e: ex[e],
                        W_gate=Wg)["out"]
    W1c = np.concatenate([ex[E][0], ex[E + 1][0]], axis=1)
    W3c = np.concatenate([ex[E][1], ex[E + 1][1]], axis=1)
    W2c = np.concatenate([ex[E][2], ex[E + 1][2]], axis=0)
    assert np.allclose(with_s - without, _torch_ffn(x, W1c, W3c, W2c),
                       rtol=1e-12, atol=1e-12)


def pin_drop_semantics(O):
    # Everything routed to expert 0 with one slot: token 0 keeps both of its
    # choices only if they fit.  With k=1 and C=1, tokens 1.. output zero.
    r = _rng(10)
    T, d, F, E = 5, 8, 8, 2
    x = r.standard_normal((T, d))
    ex = _experts(E, d, F, 100)
    bias = np.array([50.0, 0.0])
    res = O.forward(x, _shape(O, T, d, F, E, 1, cf=0.4), lambda e: ex[e],
                    W_gate=np.zeros((d, E)), bias=bias)
    assert res["capacity"] == 1
    assert np.allclose(res["out"][0], _torch_ffn(x[:1], *ex[0])[0],
                       rtol=1e-12, atol=1e-12)
    assert np.all(res["out"][1:] == 0.0)
    # k = 2, three experts: every token's first choice is expert 0 and its
    # second alternates between experts 1 and 2.  C = 3: tokens 3 and 4 lose
    # expert 0 and keep only their second expert, with the un-renormalised
    # gate.
    E = 3
    ex = _experts(E, d, F, 101)
    L = np.array([[2.0, 1.0, -1.0] if t % 2 == 0 else [2.0, -1.0, 1.0]
                  for t in range(T)])
    res = O.forward(x, _shape(O, T, d, F, E, 2, cf=0.9), lambda e: ex[e],
                    logits=L)
    assert res["capacity"] == 3
    g0 = 1.0 / (1.0 + math.exp(-1.0))
    assert np.allclose(res["w"][:, 0], g0, rtol=0, atol=1e-15)
    assert np.allclose(res["w"][:, 1], 1 - g0, rtol=0, atol=1e-15)
    y = [_torch_ffn(x, *ex[e]) for e in range(E)]
    for t in range(T):
        second = 1 if t % 2 == 0 else 2
        ref = (g0 * y[0][t] if t < 3 else 0.0) + (1 - g0) * y[second][t]
        assert np.allclose(res["out"][t], ref, rtol=1e-12, atol=1e-12)
    assert res["stats"]["dropped"] == 2
    assert list(res["dispatch"]["counts"]) == [5, 3, 2]


# ---------------------------------------------------------------- overflow
# [Routing guide] "Plain explanation" paragraph 3 names three ways to handle
# assignments beyond an expert's capacity: drop them, send them to spare
# experts, or process everything in rounds.
def pin_reroute_hand_example(O):
    # Two tokens, four experts, top-2, one slot each (2 x 2 x 0.5 / 4 = 1).
    # Token 0 takes experts 0 and 1.  Token 1 also wants 0 and 1, finds both
    # full, and its spare experts are 2 and 3 with equal scores: its first
    # overflow (a=2) goes to the lower index, 2; its second (a=3) finds 2 full
    # and goes to 3.  Both keep their own gate weights.
    L = np.array([[4.0, 3.0, 1.0, 1.0],
                  [4.0, 3.0, 2.0, 2.0]])
    assert O.capacity(2, 2, 4, 0.5) == 1
    sel, _ = O.topk_select(L, 2)
    D = O.dispatch_policy(sel, L, 4, 1, O.OVERFLOW_REROUTE)
    assert list(D["expert"]) == [0, 1, 2, 3]
    assert list(D["slot"]) == [0, 1, 2, 3]
    assert list(D["kept"]) == [1, 1, 1, 1]
    assert (D["overflowed"], D["rerouted"], D["dropped"], D["rounds"]) == (2, 2, 0, 2)
    assert list(D["counts"]) == [2, 2, 0, 0]
    # Both choices of one token overflow while a spare expert has room for
    # two rows: the token is sent there once, and its second overflow goes
    # to its next-best spare.  Three tokens, four experts, top-2, two slots
    # (3 x 2 x 4/3 / 4 = 2): tokens 0 and 1 fill experts 0 and 1; token 2's
    # first overflow (a=4) takes expert 2 (score 3 > 2), its second (a=5)
    # skips expert 2 (already its own) and takes expert 3.
    L = np.array([[4.0, 3.0, 0.0, 0.0],
                  [4.0, 3.0, 0.0, 0.0],
                  [4.0, 3.5, 3.0, 2.0]])
    assert O.capacity(3, 2, 4, 4.0 / 3.0) == 2
    sel, _ = O.topk_select(L, 2)
    D = O.dispatch_policy(sel, L, 4, 2, O.OVERFLOW_REROUTE)
    assert list(D["expert"]) == [0, 1, 0, 1, 2, 3]
    assert list(D["kept"]) == [2, 2, 1, 1]
    assert list(D["slot"]) == [0, 2, 1, 3, 4, 5]
    assert (D["overflowed"], D["rerouted"], D["dropped"]) == (2, 2, 0)
    # With expert 3 unavailable (k = 3: token 2 chose it) the second
    # overflow has no spare left and is dropped rather than doubled up.
    L3 = np.array([[4.0, 3.0, 0.0, 2.5],
                   [4.0, 3.0, 0.0, 2.5],
                   [4.0, 3.5, 3.0, 3.2]])
    sel3, _ = O.topk_select(L3, 3)
    assert [list(r) for r in sel3] == [[0, 1, 3], [0, 1, 3], [0, 1, 3]]
    D = O.dispatch_policy(sel3, L3, 4, 3, O.OVERFLOW_REROUTE)
    # every expert has 3 slots: tokens 0-2 fit on 0, 1, 3; nothing overflows
    assert D["overflowed"] == 0
    D = O.dispatch_policy(sel3, L3, 4, 2, O.OVERFLOW_REROUTE)
    # 2 slots: token 2's three choices all overflow; only expert 2 is spare
    assert list(D["expert"]) == [0, 1, 3, 0, 1, 3, 2, -1, -1]
    assert (D["overflowed"], D["rerouted"], D["dropped"]) == (3, 1, 2)
    # First choices are placed before any rerouted row: expert 2 is token 2's
    # own choice, so token 1's overflow (a=1) must skip it and take expert 1,
    # and token 3's overflow finds nothing free and is dropped.
    L = np.array([[5.0, 1.0, 1.0],
                  [5.0, 2.0, 3.0],
                  [0.0, 0.0, 6.0],
                  [5.0, 1.0, 0.0]])
    sel, _ = O.topk_select(L, 1)
    D = O.dispatch_policy(sel, L, 3, 1, O.OVERFLOW_REROUTE)
    assert list(D["expert"]) == [0, 1, 2, -1]
    assert list(D["slot"]) == [0, 1, 2, -1]
    assert list(D["perm"]) == [0, 1, 2]
    assert (D["overflowed"], D["rerouted"], D["dropped"], D["rounds"]) == (2, 1, 1, 3)
    # The same call under the other policies.
    D = O.dispatch_policy(sel, L, 3, 1, O.OVERFLOW_DROP)
    assert list(D["expert"]) == [0, -1, 2, -1] and D["dropped"] == 2
    D = O.dispatch_policy(sel, L, 3, 1, O.OVERFLOW_SEQUENTIAL)
    assert list(D["expert"]) == [0, 0, 2, 0] and D["dropped"] == 0
    assert list(D["perm"]) == [0, 1, 3, 2] and D["rounds"] == 3


def _check_reroute(O, sel, L, E, C, D):
    """Checks a rerouted dispatch against the rules it must follow, without
    recomputing it: capacity, first choices untouched, one row per token and
    expert, spare experts only, greedy best choice, drops only when full."""
    T, k = sel.shape
    flat = [int(v) for v in sel.reshape(-1)]
    base = O.dispatch(sel, E, C)
    ex = [int(v) for v in D["expert"]]
    assert np.all(D["kept"] <= C)
    assert np.array_equal(np.diff(D["offsets"]), D["kept"])
    assert int(D["kept"].sum()) + D["dropped"] == T * k
    assert D["rerouted"] + D["dropped"] == base["dropped"] == D["overflowed"]
    for a in range(T * k):
        if base["slot"][a] >= 0:                      # first choice kept
            e = flat[a]
            assert ex[a] == e
            assert D["slot"][a] - D["offsets"][e] == base["slot"][a] - base["offsets"][e]
    for e in range(E):                                # primaries lead each expert
        lo = int(D["offsets"][e])
        mine = [int(a) for a in D["perm"][lo:int(D["offsets"][e + 1])]]
        assert mine[:int(base["kept"][e])] == [int(a) for a in base["perm"][int(base["offsets"][e]):int(base["offsets"][e + 1])]]
        assert mine == sorted(mine[:int(base["kept"][e])]) + sorted(mine[int(base["kept"][e]):])
        assert all(ex[a] == e for a in mine)
    for t in range(T):                                # one row per token/expert
        placed = [ex[a] for a in range(t * k, t * k + k) if ex[a] >= 0]
        assert len(placed) == len(set(placed))
    # Occupancy of each expert just before overflow assignment a is handled:
    # its first choices plus the rerouted rows of earlier assignments.
    for a in range(T * k):
        if base["slot"][a] >= 0:
            continue
        t = a // k
        chosen = set(flat[t * k:t * k + k]) | {ex[b] for b in range(t * k, a) if ex[b] >= 0}
        occ = [int(base["kept"][c]) + sum(1 for b in range(a) if base["slot"][b] < 0 and ex[b] == c)
               for c in range(E)]
        free = [c for c in range(E) if c not in chosen and occ[c] < C]
        if ex[a] < 0:
            assert not free
        else:
            c = ex[a]
            assert c in free
            for c2 in free:                           # nothing free was better
                assert (L[t, c2], -c2) <= (L[t, c], -c)


def pin_reroute_rules(O):
    r = _rng(13)
    for (T, E, k, C) in [(40, 4, 2, 12), (33, 6, 2, 5), (64, 8, 2, 10), (25, 5, 3, 9),
                         (30, 8, 1, 2), (16, 4, 1, 1), (20, 3, 2, 7)]:
        for rep in range(3):
            L = r.standard_normal((T, E))
            L[:, 0] += 1.5
            if rep == 1:
                L = np.round(L)                      # many exact ties
            sel, _ = O.topk_select(L, k)
            D = O.dispatch_policy(sel, L, E, C, O.OVERFLOW_REROUTE)
            _check_reroute(O, sel, L, E, C, D)


def pin_reroute_degenerate(O):
    r = _rng(14)
    L = r.standard_normal((30, 4))
    L[:, 1] += 2.0
    # k = E: no token has a spare expert, so rerouting is dropping.
    sel, _ = O.topk_select(L, 4)
    a = O.dispatch_policy(sel, L, 4, 20, O.OVERFLOW_REROUTE)
    b = O.dispatch(sel, 4, 20)
    assert a["rerouted"] == 0 and a["dropped"] == b["dropped"] == 40
    assert list(a["perm"]) == list(b["perm"])
    # Room for everything: all three policies place every assignment alike.
    sel, _ = O.topk_select(L, 2)
    for pol in (O.OVERFLOW_DROP, O.OVERFLOW_REROUTE, O.OVERFLOW_SEQUENTIAL):
        D = O.dispatch_policy(sel, L, 4, 30, pol)
        assert D["dropped"] == 0 and D["overflowed"] == 0 and D["rounds"] == 1
        assert list(D["perm"]) == list(O.dispatch(sel, 4, 30)["perm"])
    # Total capacity E x C covers all T x k assignments and every token has a
    # spare expert for each overflow: nothing is dropped (T=8, k=1, C=2).
    L = np.zeros((8, 4))
    L[:, 0] = 1.0
    sel, _ = O.topk_select(L, 1)
    D = O.dispatch_policy(sel, L, 4, 2, O.OVERFLOW_REROUTE)
    assert D["dropped"] == 0 and list(D["kept"]) == [2, 2, 2, 2]
    assert list(D["expert"]) == [0, 0, 1, 1, 2, 2, 3, 3]   # ties: lowest index
    # No tokens.
    D = O.dispatch_policy(np.zeros((0, 2), np.int64), np.zeros((0, 4)), 4, 0,
                          O.OVERFLOW_REROUTE)
    assert D["rounds"] == 0 and D["dropped"] == 0 and len(D["perm"]) == 0


def pin_sequential_rounds(O):
    # Every token on expert 0 (k=1): C = ceil(T cf / E) slots, so the busiest
    # expert needs ceil(T / C) rounds; 2048 tokens, 8 experts, factor 1.25
    # give 320 slots and 7 rounds.
    for (T, E, cf, C, R) in [(2048, 8, 1.25, 320, 7), (10, 4, 1.0, 3, 4),
                             (5, 5, 1.0, 1, 5), (7, 2, 2.0, 7, 1)]:
        sel = np.zeros((T, 1), dtype=np.int64)
        L = np.zeros((T, E))
        L[:, 0] = 1.0
        assert O.capacity(T, 1, E, cf) == C
        D = O.dispatch_policy(sel, L, E, C, O.OVERFLOW_SEQUENTIAL)
        assert D["rounds"] == R and D["dropped"] == 0
        assert D["overflowed"] == T - C
        assert list(D["kept"]) == [T] + [0] * (E - 1)
        assert list(D["perm"]) == list(range(T))


def pin_overflow_forward(O):
    r = _rng(15)
    T, d, F, E, k = 24, 8, 12, 6, 2
    x = r.standard_normal((T, d))
    ex = _experts(E, d, F, 150)
    Wg = r.standard_normal((d, E))
    bias = np.array([2.0, 1.0, 0.0, 0.0, -1.0, -2.0])
    free = O.forward(x, _shape(O, T, d, F, E, k), lambda e: ex[e], W_gate=Wg,
                     bias=bias)
    # Sequential processing drops nothing: the unlimited layer, exactly.
    seq = O.forward(x, _shape(O, T, d, F, E, k, cf=0.5,
                              overflow=O.OVERFLOW_SEQUENTIAL),
                    lambda e: ex[e], W_gate=Wg, bias=bias)
    assert seq["capacity"] == 4 and seq["dispatch"]["rounds"] == 4
    assert np.array_equal(seq["out"], free["out"])
    assert seq["stats"]["dropped"] == 0
    # With identical experts the expert that runs a row does not matter: a
    # rerouted row keeps its gate weight, so a reroute that drops nothing
    # gives the unlimited layer.
    one = _experts(1, d, F, 151)[0]
    ref = O.forward(x, _shape(O, T, d, F, E, k), lambda e: one, W_gate=Wg,
                    bias=bias)
    # (At factor 1.0 every slot is needed and one token's last overflow finds
    # only the spare its first overflow took, so one assignment is dropped;
    # 1.1 leaves a slot to spare.)
    rr = O.forward(x, _shape(O, T, d, F, E, k, cf=1.1,
                             overflow=O.OVERFLOW_REROUTE),
                   lambda e: one, W_gate=Wg, bias=bias)
    D = rr["dispatch"]
    assert D["rerouted"] > 0 and D["dropped"] == 0
    assert np.allclose(rr["out"], ref["out"], rtol=1e-12, atol=1e-12)
    # Distinct experts: each token's output is the gate-weighted sum over the
    # experts that actually ran its rows.
    rr = O.forward(x, _shape(O, T, d, F, E, k, cf=0.75,
                             overflow=O.OVERFLOW_REROUTE),
                   lambda e: ex[e], W_gate=Wg, bias=bias)
    D = rr["dispatch"]
    assert D["rerouted"] > 0 and D["dropped"] > 0
    y = [_torch_ffn(x, *ex[e]) for e in range(E)]
    for t in range(T):
        want = np.zeros(d)
        for j in range(k):
            e = int(D["expert"][t * k + j])
            if e >= 0:
                want += rr["w"][t, j] * y[e][t]
        assert np.allclose(rr["out"][t], want, rtol=1e-12, atol=1e-12)
    assert rr["stats"]["dropped"] == D["dropped"]
    assert np.isclose(rr["stats"]["overflow_rate"], D["dropped"] / (T * k))


# ---------------------------------------------------------------- backward
# [Routing guide] "Plain explanation" paragraphs 2 and 4: the router learns
# through the softmax, and the auxiliary product pushes the load to balance.
def _bwd_case(O, gating, renorm, cf, overflow=None, T=14, d=6, F=8, E=5, k=2, S=1,
              seed=16):
    r = _rng(seed)
    x = r.standard_normal((T, d))
    ex = _experts(E + S, d, F, seed + 100)
    Wg = r.standard_normal((d, E)) * 0.8
    b = r.standard_normal(E) * 0.5
    b[0] += 1.0                                   # some overflow at small cf
    dout = r.standard_normal((T, d))
    shape = _shape(O, T, d, F, E, k, S=S, gating=gating, renorm=renorm, cf=cf,
                   overflow=overflow)
    return x, ex, Wg, b, dout, shape


def _loss(O, x, ex, Wg, b, dout, shape, alpha, x_router=None, beta=0.0):
    """sum(dout * out) + alpha * aux + beta * (mean router entropy), with the
    router reading x_router."""
    xr = x if x_router is None else x_router
    res = O.forward(x, shape, lambda e: ex[e], logits=O.router_logits(xr, Wg, b))
    return (float(np.sum(dout * res["out"])) + alpha * res["stats"]["aux_loss"]
            + beta * res["stats"]["entropy_token"]), res


def pin_router_backward_finite_differences(O):
    # Central differences of the layer's own forward (selection and capacity
    # decisions stay fixed: every decision margin is far above the step).
    h, alpha, beta = 1e-6, 0.7, 0.4
    for gating, renorm, cf, ovf, d in [(O.TOPK_THEN_SOFTMAX, True, 0.8, None, 6),
                                       (O.SOFTMAX_THEN_TOPK, False, 0.8, None, 6),
                                       (O.SOFTMAX_THEN_TOPK, True, 0.0, None, 6),
                                       (O.SOFTMAX_THEN_TOPK, False, 0.7, O.OVERFLOW_REROUTE, 6),
                                       (O.TOPK_THEN_SOFTMAX, True, 0.8, None, 5)]:  # d == E
        x, ex, Wg, b, dout, shape = _bwd_case(O, gating, renorm, cf, ovf, d=d)
        L0, res = _loss(O, x, ex, Wg, b, dout, shape, alpha, beta=beta)
        assert float(np.min(_full_gaps(res["logits"]))) > 5e-5   # steps move scores by ~1e-5
        if cf > 0:
            assert res["dispatch"]["overflowed"] > 0
        g = O.router_backward(x, Wg, res, shape, dout, aux_coef=alpha, entropy_coef=beta)
        for name, arr, get in (("dW_gate", Wg, lambda v: (x, ex, v, b)),
                               ("dbias", b, lambda v: (x, ex, Wg, v))):
            num = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                up, dn = arr.copy(), arr.copy()
                up[idx] += h
                dn[idx] -= h
                num[idx] = (_loss(O, *get(up), dout, shape, alpha, beta=beta)[0]
                            - _loss(O, *get(dn), dout, shape, alpha, beta=beta)[0]) / (2 * h)
            assert np.allclose(g[name], num, rtol=1e-6, atol=1e-7), (name, gating, renorm)
        # dx: the router's share only (experts keep reading the unperturbed x)
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            up, dn = x.copy(), x.copy()
            up[idx] += h
            dn[idx] -= h
            num[idx] = (_loss(O, x, ex, Wg, b, dout, shape, alpha, x_router=up, beta=beta)[0]
                        - _loss(O, x, ex, Wg, b, dout, shape, alpha, x_router=dn,
                                beta=beta)[0]) / (2 * h)
        assert np.allclose(g["dx"], num, rtol=1e-6, atol=1e-7), ("dx", gating, renorm)


def _full_gaps(L):
    return np.min(np.diff(np.sort(L, axis=1), axis=1), axis=1)


def pin_router_backward_autograd(O):
    # torch fp64 autograd of the gating with the selection held fixed.
    alpha, beta = 0.3, -0.6
    for gating, renorm in [(O.TOPK_THEN_SOFTMAX, True), (O.SOFTMAX_THEN_TOPK, False),
                           (O.SOFTMAX_THEN_TOPK, True)]:
        x, ex, Wg, b, dout, shape = _bwd_case(O, gating, renorm, 0.9, seed=17)
        _, res = _loss(O, x, ex, Wg, b, dout, shape, alpha, beta=beta)
        g = O.router_backward(x, Wg, res, shape, dout, aux_coef=alpha, entropy_coef=beta)
        T, E, k = shape.T, shape.E, shape.k
        sel = torch.as_tensor(res["sel"])
        Y = torch.zeros(T, k, shape.d, dtype=torch.float64)
        for a, y in res["yrows"].items():
            Y[a // k, a % k] = torch.as_tensor(y)
        L = torch.tensor(res["logits"], dtype=torch.float64, requires_grad=True)
        if gating == O.TOPK_THEN_SOFTMAX or renorm:
            w = torch.softmax(torch.gather(L, 1, sel), dim=1)
        else:
            w = torch.gather(torch.softmax(L, dim=1), 1, sel)
        out = (w[:, :, None] * Y).sum(1)
        f = torch.as_tensor(res["dispatch"]["counts"], dtype=torch.float64) / (T * k)
        P = torch.softmax(L, dim=1)
        aux = E * (f * P.mean(0)).sum()
        H = -(P * torch.log_softmax(L, dim=1)).sum(1).mean()
        loss = (torch.as_tensor(dout) * out).sum() + alpha * aux + beta * H
        loss.backward()
        assert np.allclose(g["dlogits"], L.grad.numpy(), rtol=1e-10, atol=1e-12)


def pin_router_backward_closed_forms(O):
    # Softmax gradients are orthogonal to a constant shift of a token's scores.
    for gating, renorm in [(O.TOPK_THEN_SOFTMAX, True), (O.SOFTMAX_THEN_TOPK, False)]:
        x, ex, Wg, b, dout, shape = _bwd_case(O, gating, renorm, 0.8, seed=18)
        _, res = _loss(O, x, ex, Wg, b, dout, shape, 0.5)
        g = O.router_backward(x, Wg, res, shape, dout, aux_coef=0.5)
        assert np.allclose(g["dlogits"].sum(axis=1), 0.0, atol=1e-12)
        dropped = [t for t in range(shape.T)
                   if all(res["dispatch"]["slot"][t * shape.k + j] < 0 for j in range(shape.k))]
        g0 = O.router_backward(x, Wg, res, shape, dout, aux_coef=0.0)
        for t in dropped:                                 # nothing ran: no gate signal
            assert np.all(g0["dlogits"][t] == 0.0)
        if gating == O.SOFTMAX_THEN_TOPK:
            # experts the token did not choose get -p_i * sum_j w_j dw_j
            for t in range(shape.T):
                s = float(np.dot(g0["dw"][t], res["w"][t]))
                for i in set(range(shape.E)) - set(int(c) for c in res["sel"][t]):
                    assert np.isclose(g0["dlogits"][t, i], -res["p"][t, i] * s, rtol=0, atol=1e-14)
    # Identical experts and Mixtral gates: the output does not depend on the
    # gates (they sum to 1), so neither does the loss.
    x, ex, Wg, b, dout, shape = _bwd_case(O, O.TOPK_THEN_SOFTMAX, True, 0.0, S=0, seed=19)
    same = [ex[0]] * shape.E
    _, res = _loss(O, x, same, Wg, b, dout, shape, 0.0)
    g = O.router_backward(x, Wg, res, shape, dout, aux_coef=0.0)
    assert np.allclose(g["dlogits"], 0.0, atol=1e-12)
    # Balanced load: each of E experts gets T/E tokens (k = 1), so f = 1/E and
    # the auxiliary gradient (E/T) p (f - <f, p>) vanishes.
    T, E = 12, 4
    L = np.full((T, E), -1.0)
    for t in range(T):
        L[t, t % E] = 2.0 + 0.1 * t
    shape = _shape(O, T, 3, 4, E, 1)
    ex = _experts(E, 3, 4, 190)
    res = O.forward(np.ones((T, 3)), shape, lambda e: ex[e], logits=L)
    g = O.router_backward(np.ones((T, 3)), np.zeros((3, E)), res, shape, np.zeros((T, 3)),
                          aux_coef=1.0)
    assert np.allclose(g["dlogits"], 0.0, atol=1e-15)
    # Equal scores: the router entropy is at its maximum ln E, so its gradient
    # vanishes.  With one dominant score, raising it lowers the entropy and
    # raising any other score raises it.
    L = np.zeros((T, E))
    res = O.forward(np.ones((T, 3)), shape, lambda e: ex[e], logits=L)
    g = O.router_backward(np.ones((T, 3)), np.zeros((3, E)), res, shape, np.zeros((T, 3)),
                          entropy_coef=1.0)
    assert np.allclose(g["dlogits"], 0.0, atol=1e-15)
    L[:, 0] = 3.0
    res = O.forward(np.ones((T, 3)), shape, lambda e: ex[e], logits=L)
    g = O.router_backward(np.ones((T, 3)), np.zeros((3, E)), res, shape, np.zeros((T, 3)),
                          entropy_coef=1.0)
    assert np.all(g["dlogits"][:, 0] < 0) and np.all(g["dlogits"][:, 1:] > 0)


def pin_router_backward_token_subset(O):
    # Rows computed for a subset of tokens equal the full computation's rows.
    x, ex, Wg, b, dout, shape = _bwd_case(O, O.SOFTMAX_THEN_TOPK, False, 0.8, seed=20)
    _, full = _loss(O, x, ex, Wg, b, dout, shape, 0.4)
    g = O.router_backward(x, Wg, full, shape, dout, aux_coef=0.4)
    toks = [0, 3, 7, shape.T - 1]
    part = O.forward(x, shape, lambda e: ex[e], logits=O.router_logits(x, Wg, b), tokens=toks)
    h = O.router_backward(x, Wg, part, shape, dout, aux_coef=0.4, tokens=toks)
    for key in ("dw", "dlogits", "dx"):
        assert np.allclose(h[key][toks], g[key][toks], rtol=1e-13, atol=1e-15), key
        rest = [t for t in range(shape.T) if t not in toks]
        assert np.all(np.isnan(h[key][rest]))


# ---------------------------------------------------------------- stats
def pin_stats_closed_forms(O):
    E, k, T = 8, 2, 64
    counts = np.full(E, T * k // E)
    p = np.full((T, E), 1.0 / E)
    st = O.routing_stats(counts, counts, p, T, k, E)
    assert abs(st["aux_loss"] - 1.0) < 1e-15
    assert abs(st["entropy_load"] - math.log(E)) < 1e-15
    assert abs(st["entropy_token"] - math.log(E)) < 1e-15
    assert st["overflow_rate"] == 0.0
    # hand example: k=1, T=4, counts [3, 1], two distinct token distributions
    p = np.array([[0.9, 0.1], [0.6, 0.4], [0.7, 0.3], [0.2, 0.8]])
    st = O.routing_stats(np.array([3, 1]), np.array([2, 1]), p, 4, 1, 2)
    P0, P1 = p.mean(0)
    assert abs(st["aux_loss"] - 2 * (0.75 * P0 + 0.25 * P1)) < 1e-15
    assert abs(st["aux_loss_kept"] - 2 * (0.5 * P0 + 0.25 * P1)) < 1e-15
    assert abs(st["overflow_rate"] - 0.25) < 1e-15
    assert abs(st["entropy_load"] - scipy.stats.entropy([0.75, 0.25])) < 1e-15
    ht = np.mean([scipy.stats.entropy(row) for row in p])
    assert abs(st["entropy_token"] - ht) < 1e-15
    # one-hot load: zero entropy (0 ln 0 = 0)
    st = O.routing_stats(np.array([4, 0, 0]), np.array([4, 0, 0]),
                         np.full((4, 3), 1 / 3), 4, 1, 3)
    assert st["entropy_load"] == 0.0


def pin_stats_skew_direction(O):
    # Concentrating both load and probability on one expert raises aux above
    # the balanced value of 1 and up to E in the limit.
    E, T, k = 4, 100, 1
    p = np.zeros((T, E))
    p[:, 0] = 1.0
    st = O.routing_stats(np.array([T, 0, 0, 0]), np.array([T, 0, 0, 0]), p,
                         T, k, E)
    assert abs(st["aux_loss"] - E) < 1e-12


def pin_active_fraction(O):
    # Without drops each token is processed by exactly k of E experts, so the
    # active share of expert parameters per token is k/E (1/4 for top-2 of 8).
    g = golden("active_fraction.json")
    E, k = g["experts"], g["top_k"]
    r = _rng(11)
    T = 200
    sel, _ = O.topk_select(r.standard_normal((T, E)), k)
    D = O.dispatch(sel, E, O.capacity(T, k, E, 0.0))
    per_token = np.zeros(T, dtype=int)
    for a in D["perm"]:
        per_token[a // k] += 1
    assert np.all(per_token == k)
    assert per_token.mean() / E == g["active_fraction"]


def pin_decode_single_token(O):
    # One token with top-2 hits exactly two experts; with DeepSeek routing
    # it hits six routed experts.
    r = _rng(12)
    for E, k in [(8, 2), (160, 6)]:
        sel, _ = O.topk_select(r.standard_normal((1, E)), k)
        D = O.dispatch(sel, E, O.capacity(1, k, E, 0.0))
        assert int((D["counts"] > 0).sum()) == k
    g = golden("deepseek_routing.json")
    assert g["top_k"] == 6 and g["shared_experts"] == 2


def pin_empty_call(O):
    res = O.forward(np.zeros((0, 8)), _shape(O, 0, 8, 8, 4, 2),
                    lambda e: _experts(1, 8, 8, 1)[0],
                    W_gate=np.zeros((8, 4)))
    assert res["out"].shape == (0, 8)
    assert res["capacity"] == 0
    assert res["stats"]["aux_loss"] == 0.0
    assert list(res["dispatch"]["counts"]) == [0, 0, 0, 0]


# ---------------------------------------------------------------- training side
# [Routing guide] "Plain explanation" paragraph 4 (router entropy high early in
# training, lower later) and "Key insights" item 3 (the load-balancing loss's
# trend is a quantity to watch).
def pin_entropy_schedule(O):
    total, high, low = 101, 0.5, 0.01
    vals = [O.entropy_schedule(s, total, high, low) for s in range(total)]
    assert vals[0] == high and abs(vals[-1] - low) <= 1e-15       # the two ends
    assert all(a > b for a, b in zip(vals, vals[1:]))             # falls every step
    assert abs(vals[50] - (high + low) / 2) <= 1e-15              # halfway: the mean
    steps = np.diff(vals)
    assert np.allclose(steps, (low - high) / (total - 1), rtol=0, atol=1e-15)   # a line
    assert O.entropy_schedule(10 ** 6, total, high, low) == vals[-1]   # held after the end
    assert O.entropy_schedule(-5, total, high, low) == high            # and before the start
    assert O.entropy_schedule(0, 1, high, low) == low


def pin_load_balance_trend_library(O):
    # the least-squares line of numpy.polyfit
    r = _rng(21)
    for n in (2, 3, 10, 57):
        v = 1.5 + r.standard_normal(n) * 0.1 - 0.02 * np.arange(n)
        res = O.load_balance_trend(list(v))
        slope, intercept = np.polyfit(np.arange(n), v, 1)
        assert abs(res["slope"] - slope) <= 1e-12 * max(1.0, abs(slope))
        assert abs(res["mean"] - float(np.mean(v))) <= 1e-14
        assert res["last"] == v[-1] and res["n"] == n


def pin_load_balance_trend_closed_forms(O):
    # an exact line gives its own slope; a constant (perfect balance, aux = 1
    # every step) gives 0; adding a constant changes nothing; two points give
    # their difference
    assert abs(O.load_balance_trend([3.0 - 0.25 * i for i in range(9)])["slope"] + 0.25) <= 1e-15
    assert O.load_balance_trend([1.0] * 7)["slope"] == 0.0
    a = O.load_balance_trend([1.2, 1.7, 1.1, 1.4])["slope"]
    b = O.load_balance_trend([11.2, 11.7, 11.1, 11.4])["slope"]
    assert abs(a - b) <= 1e-12
    assert O.load_balance_trend([2.0, 1.5])["slope"] == -0.5
    try:
        O.load_balance_trend([1.0])
    except ValueError:
        pass
    else:
        raise AssertionError("a single value has no trend")


def pin_load_balance_trend_of_balancing_routing(O):
    # Batches whose router bias toward expert 0 shrinks step by step (the
    # load evening out): the aux loss of each batch (routing_stats) falls
    # toward 1, so its trend is negative; with the bias growing it is
    # positive.
    r = _rng(22)
    T, E, k = 400, 8, 2
    def aux_of(bias0):
        L = r.standard_normal((T, E))
        L[:, 0] += bias0
        sel, _ = O.topk_select(L, k)
        D = O.dispatch(sel, E, T)
        return O.routing_stats(D["counts"], D["kept"], O.softmax_all(L), T, k, E)["aux_loss"]
    falling = [aux_of(b) for b in np.linspace(3.0, 0.0, 12)]
    rising = [aux_of(b) for b in np.linspace(0.0, 3.0, 12)]
    assert O.load_balance_trend(falling)["slope"] < 0 < O.load_balance_trend(rising)["slope"]
    assert abs(falling[-1] - 1.0) < 0.1


ALL_PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
