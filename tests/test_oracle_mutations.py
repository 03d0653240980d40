"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin catches each.  This is evidence that the pins constrain every step of
the oracle, not only that the oracle agrees with itself."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle.oracle as O
import pins

_orig = {name: getattr(O, name) for name in dir(O) if not name.startswith("__")}


def _drop_earliest(sel, E, C):
    # keeps the LATEST C assignments per expert instead of the earliest
    T, k = sel.shape
    rev = sel.reshape(-1)[::-1].reshape(T, k)
    D = _orig["dispatch"](rev, E, C)
    n = T * k
    slot = D["slot"][::-1].copy()
    perm = np.array([n - 1 - a for a in D["perm"]], dtype=np.int64)
    D.update(slot=slot, perm=perm)
    return D


def _silu_on_w3(X, W1, W3, W2):
    return _orig["expert_ffn"](X, W3, W1, W2)


def _w2_transposed(X, W1, W3, W2):
    X = np.asarray(X, dtype=np.float64)
    h = O.silu(X @ np.asarray(W1, np.float64)) * (X @ np.asarray(W3, np.float64))
    W2 = np.asarray(W2, np.float64)
    return h @ (W2.T if W2.shape[0] == W2.shape[1] else W2)


def _router_transposed(x, W_gate, bias=None):
    W = np.asarray(W_gate, np.float64)
    return _orig["router_logits"](x, W.T if W.shape[0] == W.shape[1] else W, bias)


def _router_bias_sign(x, W_gate, bias=None):
    return _orig["router_logits"](x, W_gate, None if bias is None else -np.asarray(bias))


def _topk_high_index(logits, k):
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    sel = np.empty((T, k), dtype=np.int64)
    margin = np.full(T, np.inf)
    for t in range(T):
        order = sorted(range(E), key=lambda i: (-logits[t, i], -i))
        sel[t] = order[:k]
    return sel, margin


def _topk_signed_zero_order(logits, k):
    # sorts with -0.0 below +0.0 (the sortable-integer trick)
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    sel = np.empty((T, k), dtype=np.int64)
    margin = np.full(T, np.inf)
    for t in range(T):
        key = lambda i: (-(logits[t, i] + (0.0 if math.copysign(1, logits[t, i]) > 0 else -1e-300)), i)  # noqa
        order = sorted(range(E), key=key)
        sel[t] = order[:k]
        top = [logits[t, i] for i in order[:min(k + 1, E)]]
        for a, b in zip(top[:-1], top[1:]):
            margin[t] = min(margin[t], a - b)
    return sel, margin


def _gates_all_softmax(logits, sel, gating, renormalize):
    return _orig["gate_weights"](logits, sel, O.SOFTMAX_THEN_TOPK, False)


def _gates_renormalised_b(logits, sel, gating, renormalize):
    return _orig["gate_weights"](logits, sel, gating, True)


def _capacity_floor(T, k, E, cf):
    if cf is None or cf <= 0:
        return int(T)
    return int(math.floor(Fraction(T * k) * Fraction(repr(float(cf))) / E))


def _capacity_binary(T, k, E, cf):
    if cf is None or cf <= 0:
        return int(T)
    return int(math.ceil(T * k * cf / E))


def _capacity_no_k(T, k, E, cf):
    return _orig["capacity"](T, 1, E, cf)


def _stats_no_E(counts, kept, p, T, k, E):
    st = _orig["routing_stats"](counts, kept, p, T, k, E)
    if T:
        st["aux_loss"] /= E
    return st


def _stats_post_drop_f(counts, kept, p, T, k, E):
    return _orig["routing_stats"](kept, kept, p, T, k, E)


def _stats_entropy_sign(counts, kept, p, T, k, E):
    st = _orig["routing_stats"](counts, kept, p, T, k, E)
    st["entropy_token"] = -st["entropy_token"]
    return st


def _softmax_no_shift_bug(logits):
    # forgets to normalise
    z = np.asarray(logits, np.float64)
    return np.exp(z - z.max(axis=1, keepdims=True))


def _forward_no_shared(x, shape, expert_weights, **kw):
    from dataclasses import replace
    return _orig["forward"](x, replace(shape, S=0), expert_weights, **kw)


def _forward_renorm_after_drop(x, shape, expert_weights, **kw):
    res = _orig["forward"](x, shape, expert_weights, **kw)
    # rescale each token's routed part by 1 / (sum of kept gates)
    k = shape.k
    slot = res["dispatch"]["slot"].reshape(-1, k)
    kept_w = np.where(slot >= 0, res["w"], 0.0).sum(1)
    if shape.S == 0:
        scale = np.where(kept_w > 0, 1.0 / np.where(kept_w > 0, kept_w, 1), 1)
        res["out"] = res["out"] * scale[:, None]
    return res


def _ffn_relu(X, W1, W3, W2):
    X = np.asarray(X, dtype=np.float64)
    u = X @ np.asarray(W1, np.float64)
    h = np.maximum(u, 0) * (X @ np.asarray(W3, np.float64))
    return h @ np.asarray(W2, np.float64)


def _reroute_variant(mode):
    """A rerouting dispatch built on the drop dispatch with one planted
    mistake: 'high' breaks score ties to the higher index, 'own' lets an
    overflow land on another of the token's own choices, 'worst' takes the
    lowest-scoring spare expert, 'onepass' handles assignments strictly in
    flat order so a later first choice can find its slot taken, 'weightless'
    runs rerouted rows but leaves them out of the combine, 'twice' lets a
    token's second overflow land on the spare expert its first one took."""
    def fn(sel, logits, E, C, policy=O.OVERFLOW_DROP):
        if policy != O.OVERFLOW_REROUTE:
            return _orig["dispatch_policy"](sel, logits, E, C, policy)
        T, k = sel.shape
        flat = [int(v) for v in sel.reshape(-1)]
        D = _orig["dispatch"](sel, E, C)
        fill = [0] * E
        expert = [-1] * len(flat)
        primary = [r < C for r in D["rank"]]
        if mode == "onepass":
            primary = [False] * len(flat)
        for a, e in enumerate(flat):
            if primary[a]:
                expert[a] = e
                fill[e] += 1
        for a, e in enumerate(flat):
            if primary[a]:
                continue
            if mode == "onepass" and fill[e] < C:
                expert[a] = e
                fill[e] += 1
                continue
            t = a // k
            chosen = set(flat[t * k:(t + 1) * k])
            if mode != "twice":
                chosen.update(expert[b] for b in range(t * k, a) if expert[b] >= 0)
            cand = [c for c in range(E) if fill[c] < C and (mode == "own" or c not in chosen)]
            if mode == "own":
                cand = [c for c in cand if c != e]
            if not cand:
                continue
            key = {"high": lambda c: (logits[t, c], c),
                   "worst": lambda c: (-logits[t, c], -c)}.get(mode, lambda c: (logits[t, c], -c))
            best = max(cand, key=key)
            expert[a] = best
            fill[best] += 1
        offsets = np.concatenate([[0], np.cumsum(fill)]).astype(np.int64)
        slot = np.full(len(flat), -1, dtype=np.int64)
        perm = []
        for e in range(E):
            first = [a for a in range(len(flat)) if expert[a] == e and flat[a] == e and (primary[a] or mode == "onepass")]
            rest = [a for a in range(len(flat)) if expert[a] == e and a not in first]
            for a in first + rest:
                slot[a] = len(perm)
                perm.append(a)
        moved = sum(1 for a in range(len(flat)) if expert[a] >= 0 and expert[a] != flat[a])
        over = int(D["dropped"])
        out = dict(D)
        out.update(kept=np.array(fill, dtype=np.int64), offsets=offsets, slot=slot,
                   perm=np.array(perm, dtype=np.int64), expert=np.array(expert, dtype=np.int64),
                   overflowed=over, rerouted=moved, dropped=len(flat) - sum(fill),
                   rounds=_orig["dispatch_policy"](sel, logits, E, C, O.OVERFLOW_DROP)["rounds"])
        if mode == "weightless":
            keep = [a for a in perm if expert[a] == flat[a]]
            out["perm"] = np.array(keep, dtype=np.int64)
            out["offsets"] = np.concatenate([[0], np.cumsum(
                [sum(1 for a in keep if expert[a] == e) for e in range(E)])]).astype(np.int64)
        return out
    return fn


def _sequential_as_drop(sel, logits, E, C, policy=O.OVERFLOW_DROP):
    if policy == O.OVERFLOW_SEQUENTIAL:
        policy = O.OVERFLOW_DROP
    return _orig["dispatch_policy"](sel, logits, E, C, policy)


def _rounds_floor(sel, logits, E, C, policy=O.OVERFLOW_DROP):
    D = _orig["dispatch_policy"](sel, logits, E, C, policy)
    D["rounds"] = max([int(c) // max(C, 1) for c in D["counts"]], default=0)
    return D


def _bwd_variant(mode):
    """The router backward with one planted mistake: 'dropped' gives dropped
    assignments their expert's dot product anyway, 'selected_only' drops the
    softmax signal to unchosen experts, 'aux_no_E' loses the factor E,
    'aux_sign' flips the auxiliary term, 'dx_untransposed' multiplies by
    W_gate instead of its transpose (shapes allowing), 'dw_unweighted' leaves
    out the gate weight in the chosen-softmax Jacobian."""
    def fn(x, W_gate, fwd, shape, dout, aux_coef=0.0, tokens=None, entropy_coef=0.0):
        if tokens is not None:   # the planted mistakes live in the full computation
            return _orig["router_backward"](x, W_gate, fwd, shape, dout, aux_coef, tokens,
                                            entropy_coef)
        T, E, k = shape.T, shape.E, shape.k
        g = _orig["router_backward"](x, W_gate, fwd, shape, dout, aux_coef,
                                     entropy_coef=entropy_coef)
        if mode == "dropped":
            fwd2 = dict(fwd)
            yr = dict(fwd["yrows"])
            for a in range(T * k):
                if a not in yr:
                    yr[a] = np.ones(shape.d)
            fwd2["yrows"] = yr
            return _orig["router_backward"](x, W_gate, fwd2, shape, dout, aux_coef,
                                            entropy_coef=entropy_coef)
        if mode == "selected_only":
            dl = g["dlogits"].copy()
            for t in range(T):
                keep = set(int(c) for c in fwd["sel"][t])
                for i in range(E):
                    if i not in keep:
                        dl[t, i] = 0.0
        elif mode in ("ent_sign", "ent_no_H", "ent_no_T"):
            g0 = _orig["router_backward"](x, W_gate, fwd, shape, dout, aux_coef)
            part = g["dlogits"] - g0["dlogits"]
            if mode == "ent_sign":
                dl = g0["dlogits"] - part
            elif mode == "ent_no_T":
                dl = g0["dlogits"] + part * T
            else:   # drops the + H_t inside the bracket: -p ln p only
                p = fwd["p"]
                with np.errstate(divide="ignore", invalid="ignore"):
                    lnp = np.where(p > 0, np.log(p), 0.0)
                dl = g0["dlogits"] + entropy_coef / T * (-p * lnp)
        elif mode in ("aux_no_E", "aux_sign"):
            g0 = _orig["router_backward"](x, W_gate, fwd, shape, dout, 0.0,
                                          entropy_coef=entropy_coef)
            aux_part = g["dlogits"] - g0["dlogits"]
            dl = g0["dlogits"] + (aux_part / E if mode == "aux_no_E" else -aux_part)
        elif mode == "dx_untransposed":
            W = np.asarray(W_gate, np.float64)
            g["dx"] = g["dlogits"] @ (W if W.shape[0] == W.shape[1] else W.T)
            return g
        elif mode == "dw_unweighted":
            dl = g["dlogits"].copy()
            w = fwd["w"]
            for t in range(T):
                s = float(np.dot(w[t], g["dw"][t]))
                for j in range(k):
                    dl[t, fwd["sel"][t, j]] = g["dw"][t, j] - s
        x64 = np.asarray(x, np.float64)
        return dict(dw=g["dw"], dlogits=dl, dW_gate=x64.T @ dl, dbias=dl.sum(0),
                    dx=dl @ np.asarray(W_gate, np.float64).T)
    return fn


def _schedule_reversed(step, total_steps, high, low):
    # rises from low to high instead of falling
    return _orig["entropy_schedule"](step, total_steps, low, high)


def _schedule_unclamped(step, total_steps, high, low):
    if total_steps <= 1:
        return float(low)
    return float(high) + (float(low) - float(high)) * int(step) / (int(total_steps) - 1)


def _trend_sign(values):
    res = _orig["load_balance_trend"](values)
    res["slope"] = -res["slope"]
    return res


def _trend_endpoints(values):
    # the slope between the first and last value instead of the fitted line
    res = _orig["load_balance_trend"](values)
    res["slope"] = (float(values[-1]) - float(values[0])) / (len(values) - 1)
    return res


def _trend_unnormalised(values):
    # the covariance without dividing by the spread of the step numbers
    res = _orig["load_balance_trend"](values)
    n = len(values)
    m = (n - 1) / 2.0
    res["slope"] = res["slope"] * sum((i - m) ** 2 for i in range(n)) / n
    return res


MUTATIONS = {
    "schedule_rises": ("entropy_schedule", _schedule_reversed),
    "schedule_not_held_at_ends": ("entropy_schedule", _schedule_unclamped),
    "trend_sign": ("load_balance_trend", _trend_sign),
    "trend_endpoints_only": ("load_balance_trend", _trend_endpoints),
    "trend_unnormalised": ("load_balance_trend", _trend_unnormalised),
    "bwd_dropped_rows_counted": ("router_backward", _bwd_variant("dropped")),
    "bwd_no_signal_to_unchosen": ("router_backward", _bwd_variant("selected_only")),
    "bwd_aux_without_E": ("router_backward", _bwd_variant("aux_no_E")),
    "bwd_aux_sign": ("router_backward", _bwd_variant("aux_sign")),
    "bwd_dx_untransposed": ("router_backward", _bwd_variant("dx_untransposed")),
    "bwd_jacobian_unweighted": ("router_backward", _bwd_variant("dw_unweighted")),
    "bwd_entropy_sign": ("router_backward", _bwd_variant("ent_sign")),
    "bwd_entropy_without_H": ("router_backward", _bwd_variant("ent_no_H")),
    "bwd_entropy_without_1_over_T": ("router_backward", _bwd_variant("ent_no_T")),
    "reroute_ties_to_high_index": ("dispatch_policy", _reroute_variant("high")),
    "reroute_onto_own_choice": ("dispatch_policy", _reroute_variant("own")),
    "reroute_to_worst_spare": ("dispatch_policy", _reroute_variant("worst")),
    "reroute_single_pass": ("dispatch_policy", _reroute_variant("onepass")),
    "reroute_rows_not_combined": ("dispatch_policy", _reroute_variant("weightless")),
    "reroute_same_spare_twice": ("dispatch_policy", _reroute_variant("twice")),
    "sequential_drops": ("dispatch_policy", _sequential_as_drop),
    "rounds_rounded_down": ("dispatch_policy", _rounds_floor),
    "dispatch_drops_earliest": ("dispatch", _drop_earliest),
    "silu_on_w3_branch": ("expert_ffn", _silu_on_w3),
    "w2_transposed": ("expert_ffn", _w2_transposed),
    "ffn_relu": ("expert_ffn", _ffn_relu),
    "router_transposed": ("router_logits", _router_transposed),
    "router_bias_sign": ("router_logits", _router_bias_sign),
    "topk_ties_to_high_index": ("topk_select", _topk_high_index),
    "topk_signed_zero_ordered": ("topk_select", _topk_signed_zero_order),
    "mixtral_gates_over_all": ("gate_weights", _gates_all_softmax),
    "deepseek_gates_renormalised": ("gate_weights", _gates_renormalised_b),
    "capacity_floor": ("capacity", _capacity_floor),
    "capacity_binary_double": ("capacity", _capacity_binary),
    "capacity_without_k": ("capacity", _capacity_no_k),
    "aux_without_E": ("routing_stats", _stats_no_E),
    "aux_post_drop_fraction": ("routing_stats", _stats_post_drop_f),
    "entropy_sign": ("routing_stats", _stats_entropy_sign),
    "softmax_unnormalised": ("softmax_all", _softmax_no_shift_bug),
    "shared_experts_skipped": ("forward", _forward_no_shared),
    "renormalise_after_drop": ("forward", _forward_renorm_after_drop),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(O)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutation {name}"
