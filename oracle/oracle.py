"""fp64 CPU oracle for the forward pass of a sparse mixture-of-experts FFN layer
with a per-expert capacity limit.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header, table
or helper with the HIP library and imports nothing from it.

It is written to be slow and obviously right.  Every step follows the order in
which the pages walk a token through the layer, and every function names the
passage it restates.  Page titles used in the citations:

* [Mixtral explainer]  "Mixtral 8x7B and MoE explained: sparse mixture of
  experts, two experts per token" (allinfo.ai.kr)
* [MoE explained]      "Mixture-of-experts models, explained simply"
  (welclai.com)
* [MoE wiki]           "Mixture of experts" (wikiprompt.org)
* [Routing guide]      "MoE routing, fully explained: Mixtral/DeepSeek
  structure, load balancing, capacity factor" (allinfo.ai.kr)

Sections of the allinfo.ai.kr pages are "Key messages", "Plain explanation"
(paragraphs numbered from 1) and "Key insights".

Precision: everything is float64.  bf16 or fp32 inputs are widened exactly.
No intermediate is rounded.  The matrix products use ``numpy.matmul`` (a library
primitive); routing and dispatch are explicit loops in token order.

Readings taken where the pages leave a step open (each one also listed in the
design notes):

* top-k ties go to the lower expert index; -0.0 equals +0.0 (IEEE compare);
* capacity C = ceil(T*k*cf/E) computed exactly on the decimal value of cf;
  with no limit (cf <= 0) C = T, the most one expert can ever receive;
* overflow is dropped latest-first in flat assignment order a = t*k + j;
* a dropped assignment contributes zero and the surviving gates are NOT
  renormalised; a token with every assignment dropped outputs only the
  shared-expert sum (zero without shared experts);
* expert FFN is SwiGLU with silu on the W1 branch: (silu(x W1) * (x W3)) W2;
* shared experts are added with gate 1;
* load-balance statistics use pre-drop fractions f_i = count_i/(T*k) and the
  mean full softmax P_i over all E experts in both gating modes;
* "routing entropy" is reported two ways: entropy of the expert-load
  distribution and the mean per-token router entropy, both in nats;
* overflow policies other than dropping: a rerouted assignment goes, after
  every first choice has taken its slot and in flat assignment order, to the
  best-scoring expert (ties to the lower index) that the token did not choose
  and has not been sent to already, and that still has a free slot, and
  keeps its gate weight; with sequential
  processing nothing is dropped, the output equals the unlimited layer's, and
  the number of capacity-sized rounds of the busiest expert is reported;
* the router backward differentiates the gates, the softmax and the
  auxiliary product; the top-k selection, the capacity decisions and the
  load fractions f_i are held fixed (they are piecewise constant).

Nothing here is "parity unpinned": every function is checked by
``tests/test_oracle_pins.py`` against page values, closed forms, library
routines or brute force.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from fractions import Fraction
from typing import Callable, Optional, Sequence

import numpy as np

TOPK_THEN_SOFTMAX = 0  # Mixtral-style gating
SOFTMAX_THEN_TOPK = 1  # DeepSeek-style gating


# Overflow policies.  [Routing guide] "Plain explanation" paragraph 3: an
# expert takes a fixed number of tokens per batch, and what exceeds it can
# only be dropped (fast, costs quality), sent to spare experts (blurs
# specialisation, costs coordination) or processed in full, round after round
# (costs latency).
OVERFLOW_DROP = 0
OVERFLOW_REROUTE = 1
OVERFLOW_SEQUENTIAL = 2


@dataclass(frozen=True)
class LayerShape:
    """Shape and routing options of one MoE layer call."""

    T: int          # tokens in this call (the "batch" of the capacity formula)
    d: int          # model width
    F: int          # expert hidden width
    E: int          # routed experts
    k: int          # experts kept per token
    S: int = 0      # always-on shared experts
    gating: int = TOPK_THEN_SOFTMAX
    renormalize: bool = True
    capacity_factor: float = 0.0   # <= 0: no limit
    overflow: int = OVERFLOW_DROP


# ---------------------------------------------------------------------------
# Capacity.  [Routing guide] "Plain explanation" paragraph 5: the per-expert
# buffer is about batch x top-k x capacity factor / number of experts; the
# page works 2048 tokens, 8 experts, top-2, factor 1.25 to about 640 slots.
# ---------------------------------------------------------------------------
def capacity(T: int, k: int, E: int, capacity_factor: float) -> int:
    """Token slots per expert.

    The pages give the formula only approximately; the reading here rounds up
    the exact rational value, taking the capacity factor as the decimal number
    it is written as (1.1 means 11/10, not the nearest binary double).
    Without a limit the capacity is T: one token never selects one expert twice.
    """
    if capacity_factor is None or capacity_factor <= 0:
        return int(T)
    cf = Fraction(repr(float(capacity_factor)))
    q = Fraction(int(T) * int(k)) * cf / int(E)
    return int(math.ceil(q))


# ---------------------------------------------------------------------------
# Router.  [Mixtral explainer] "Plain explanation" paragraph 3 and [Routing
# guide] "Plain explanation" paragraph 2: a small learned network scores every
# expert for each token, like a classifier producing one logit per class.
# ---------------------------------------------------------------------------
def router_logits(x: np.ndarray, W_gate: np.ndarray,
                  bias: Optional[np.ndarray] = None) -> np.ndarray:
    """logits[t, i] = sum_c x[t, c] * W_gate[c, i] (+ bias[i]), in float64.

    W_gate is stored [d, E] (input dimension first).  The optional bias is the
    per-expert logit offset of the skewed-routing workload; it is added before
    any selection, gating or statistic sees the logits.
    """
    x64 = np.asarray(x, dtype=np.float64)
    w64 = np.asarray(W_gate, dtype=np.float64)
    logits = np.matmul(x64, w64)
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    return logits


# ---------------------------------------------------------------------------
# Top-k selection.  [Mixtral explainer] "Plain explanation" paragraph 3 keeps
# the two highest-scoring of eight experts; [Routing guide] "Plain explanation"
# paragraphs 2 and 4 keep the top k (two for Mixtral, six for DeepSeek V2).
# ---------------------------------------------------------------------------
def topk_select(logits: np.ndarray, k: int):
    """Per token, the k experts with the largest logits, best first.

    Experts are ordered by (logit descending, index ascending).  Python's
    tuple comparison uses IEEE equality on floats, so -0.0 and +0.0 tie and the
    lower index wins.  Also returns, per token, the smallest gap between
    neighbours among the top min(k+1, E) sorted logits: the margin by which
    both the chosen set and its order are decided.
    """
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    if not np.all(np.isfinite(logits)):
        raise ValueError("router logits must be finite")
    sel = np.empty((T, k), dtype=np.int64)
    margin = np.full(T, np.inf)
    for t in range(T):
        row = logits[t]
        order = sorted(range(E), key=lambda i: (-row[i], i))
        sel[t] = order[:k]
        top = [row[i] for i in order[:min(k + 1, E)]]
        for a, b in zip(top[:-1], top[1:]):
            margin[t] = min(margin[t], a - b)
    return sel, margin


def softmax_all(logits: np.ndarray) -> np.ndarray:
    """Probability over all E experts per token ([Routing guide] "Plain
    explanation" paragraph 2: the router produces a distribution over every
    expert).  Shifted by the row maximum before exponentiating."""
    logits = np.asarray(logits, dtype=np.float64)
    z = logits - logits.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------------------
# Gate weights.
#   Mixtral style ([Mixtral explainer] "Plain explanation" paragraph 3):
#     softmax taken over the k selected logits only.
#   DeepSeek style ([Routing guide] "Plain explanation" paragraphs 2 and 4):
#     softmax over all experts first, then the top-k probabilities are used;
#     the DeepSeek-shaped workload keeps them without renormalising.
# ---------------------------------------------------------------------------
def gate_weights(logits: np.ndarray, sel: np.ndarray, gating: int,
                 renormalize: bool) -> np.ndarray:
    logits = np.asarray(logits, dtype=np.float64)
    T, k = sel.shape
    w = np.empty((T, k), dtype=np.float64)
    if gating == TOPK_THEN_SOFTMAX:
        for t in range(T):
            chosen = logits[t, sel[t]]
            e = np.exp(chosen - chosen[0])   # chosen[0] is the largest
            w[t] = e / e.sum()
    elif gating == SOFTMAX_THEN_TOPK:
        p = softmax_all(logits)
        for t in range(T):
            w[t] = p[t, sel[t]]
            if renormalize:
                w[t] = w[t] / w[t].sum()
    else:
        raise ValueError(f"unknown gating mode {gating}")
    return w


# ---------------------------------------------------------------------------
# Dispatch with a capacity limit.  [Routing guide] "Plain explanation"
# paragraph 3: each expert takes a fixed number of tokens per batch and the
# simplest overflow policy drops the excess; paragraph 5 sizes the buffer.
# ---------------------------------------------------------------------------
def dispatch(sel: np.ndarray, E: int, C: int) -> dict:
    """Assign every (token, choice) pair a slot in its expert's buffer.

    Assignments are visited in flat order a = t*k + j.  rank[a] counts the
    earlier assignments to the same expert; the assignment is kept when
    rank < C.  Kept rows of expert e occupy slots offsets[e] .. offsets[e+1]-1
    in visiting order; perm[slot] gives back the assignment.  Dropped
    assignments get slot -1.
    """
    T, k = sel.shape
    flat = [int(v) for v in sel.reshape(-1)]
    seen = [0] * E
    rank = [0] * len(flat)
    for a, e in enumerate(flat):
        rank[a] = seen[e]
        seen[e] += 1
    counts = np.array(seen, dtype=np.int64)
    kcount = np.minimum(counts, C)
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + kcount[e]
    slot = np.full(len(flat), -1, dtype=np.int64)
    perm = np.full(int(offsets[E]), -1, dtype=np.int64)
    for a, e in enumerate(flat):
        if rank[a] < C:
            s = int(offsets[e]) + rank[a]
            slot[a] = s
            perm[s] = a
    return dict(counts=counts, kept=kcount, offsets=offsets,
                rank=np.array(rank, dtype=np.int64), slot=slot, perm=perm,
                dropped=int(np.sum(counts - kcount)), capacity=int(C))


def dispatch_policy(sel: np.ndarray, logits: np.ndarray, E: int, C: int,
                    policy: int = OVERFLOW_DROP) -> dict:
    """Slots under one of the overflow policies of [Routing guide] "Plain
    explanation" paragraph 3.  Returns what ``dispatch`` returns, plus
    ``expert`` (the expert that processes each assignment, -1 if dropped),
    ``overflowed`` (assignments that found their chosen expert full),
    ``rerouted`` (of those, the ones a spare expert took) and ``rounds`` (the
    capacity-sized rounds the busiest chosen expert needs; 0 for no tokens).

    * drop: ``dispatch`` as it is;
    * sequential: every assignment is processed by its chosen expert, in
      rounds of C rows, so nothing is dropped;
    * reroute: first choices take slots as in ``dispatch``; then every
      assignment that found its expert full, in flat order a = t*k + j, goes
      to the best-scoring expert of token t (ties to the lower index) among
      those that t did not choose, that t's earlier assignments were not
      sent to, and that still have a free slot, after the rows already
      there; with no such expert it is dropped.
    """
    T, k = sel.shape
    d = dispatch(sel, E, C)
    flat = [int(v) for v in sel.reshape(-1)]
    rank = [int(r) for r in d["rank"]]
    overflowed = sum(1 for r in rank if r >= C)
    rounds = max([-(-int(c) // C) for c in d["counts"] if c > 0], default=0)
    if policy == OVERFLOW_SEQUENTIAL:
        full = dispatch(sel, E, max(T, 1))    # no token picks an expert twice
        full.update(capacity=int(C), expert=np.asarray(flat, dtype=np.int64),
                    overflowed=overflowed, rerouted=0, rounds=rounds)
        return full
    expert = np.array([e if r < C else -1 for e, r in zip(flat, rank)],
                      dtype=np.int64)
    d.update(expert=expert, overflowed=overflowed, rerouted=0, rounds=rounds)
    if policy == OVERFLOW_DROP or overflowed == 0:
        return d
    if policy != OVERFLOW_REROUTE:
        raise ValueError(f"unknown overflow policy {policy}")

    scores = np.asarray(logits, dtype=np.float64)
    fill = [int(v) for v in d["kept"]]        # rows per expert so far
    extra = [[] for _ in range(E)]            # rerouted assignments, in order
    for a in range(len(flat)):
        if expert[a] >= 0:
            continue
        t = a // k
        # a token is never sent to one expert twice: its own choices and the
        # spare experts its earlier assignments were sent to are excluded
        chosen = set(flat[t * k:(t + 1) * k])
        chosen.update(int(expert[b]) for b in range(t * k, a) if expert[b] >= 0)
        best = -1
        for c in range(E):
            if c in chosen or fill[c] >= C:
                continue
            if best < 0 or scores[t, c] > scores[t, best]:
                best = c                      # strict >: a tie keeps the lower index
        if best >= 0:
            expert[a] = best
            extra[best].append(a)
            fill[best] += 1

    kept = np.array(fill, dtype=np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + kept[e]
    slot = np.full(len(flat), -1, dtype=np.int64)
    perm = np.full(int(offsets[E]), -1, dtype=np.int64)
    for a, e in enumerate(flat):              # first choices keep their places
        if rank[a] < C:
            slot[a] = offsets[e] + rank[a]
            perm[slot[a]] = a
    for e in range(E):                        # rerouted rows follow them
        for i, a in enumerate(extra[e]):
            slot[a] = offsets[e] + int(d["kept"][e]) + i
            perm[slot[a]] = a
    rerouted = sum(len(x) for x in extra)
    d.update(kept=kept, offsets=offsets, slot=slot, perm=perm,
             rerouted=rerouted, dropped=overflowed - rerouted)
    return d


# ---------------------------------------------------------------------------
# Expert FFN.  [Mixtral explainer] "Plain explanation" paragraph 2: the
# feed-forward block widens the token vector (about 4k) to a hidden width
# (about 14k) and back, token by token.  The gated SwiGLU form is the
# workload's choice; the pages do not name the activation.
# ---------------------------------------------------------------------------
def silu(u: np.ndarray) -> np.ndarray:
    """u * sigmoid(u), written as u / (1 + exp(-u))."""
    with np.errstate(over="ignore"):
        return u / (1.0 + np.exp(-u))


def expert_ffn(X: np.ndarray, W1: np.ndarray, W3: np.ndarray,
               W2: np.ndarray) -> np.ndarray:
    """(silu(X W1) * (X W3)) W2 for rows X [n, d]; W1, W3 [d, F]; W2 [F, d]."""
    X = np.asarray(X, dtype=np.float64)
    u = np.matmul(X, np.asarray(W1, dtype=np.float64))
    v = np.matmul(X, np.asarray(W3, dtype=np.float64))
    h = silu(u) * v
    return np.matmul(h, np.asarray(W2, dtype=np.float64))


# ---------------------------------------------------------------------------
# Load-balance and routing statistics.  [Routing guide] "Plain explanation"
# paragraph 4: per expert, multiply the fraction of tokens it actually got by
# the total probability the router gave it, and sum; "Key insights" item 3
# lists per-expert token counts, overflow rate and routing entropy among the
# quantities to watch.
# ---------------------------------------------------------------------------
def routing_stats(counts: np.ndarray, kept: np.ndarray, p: np.ndarray,
                  T: int, k: int, E: int) -> dict:
    """aux = E * sum_i f_i * P_i with f_i = count_i / (T k) (before drops) and
    P_i the mean over tokens of the full softmax.  It equals 1 when both are
    uniform.  Also: overflow rate = dropped / (T k); entropy of the load
    distribution f (0 ln 0 = 0); mean per-token entropy of p.  All in nats.
    An empty call (T = 0) reports zeros."""
    counts = np.asarray(counts, dtype=np.int64)
    kept = np.asarray(kept, dtype=np.int64)
    n_assign = T * k
    dropped = int(np.sum(counts - kept))
    if T == 0:
        return dict(aux_loss=0.0, aux_loss_kept=0.0, overflow_rate=0.0,
                    entropy_load=0.0, entropy_token=0.0, dropped=0,
                    assignments=0, P=np.zeros(E))
    f = counts.astype(np.float64) / n_assign
    f_kept = kept.astype(np.float64) / n_assign
    P = np.asarray(p, dtype=np.float64).mean(axis=0)
    aux = E * float(np.sum(f * P))
    aux_kept = E * float(np.sum(f_kept * P))
    h_load = 0.0
    for fi in f:
        if fi > 0:
            h_load -= fi * math.log(fi)
    pt = np.asarray(p, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        terms = np.where(pt > 0, pt * np.log(pt), 0.0)
    h_tok = float(np.mean(-terms.sum(axis=1)))
    return dict(aux_loss=aux, aux_loss_kept=aux_kept,
                overflow_rate=dropped / n_assign, entropy_load=h_load,
                entropy_token=h_tok, dropped=dropped, assignments=n_assign,
                P=P)


# ---------------------------------------------------------------------------
# The whole layer.  [Routing guide] "Plain explanation" paragraphs 2-5 and
# [MoE wiki] "How it works": score, keep top-k, handle overflow, run only the
# chosen experts, take the gate-weighted sum; [Routing guide] paragraph 4 adds
# always-on shared experts (DeepSeek V2: two shared plus top-6 routed).
# ---------------------------------------------------------------------------
ExpertWeights = Callable[[int], Sequence[np.ndarray]]


def forward(x: np.ndarray, shape: LayerShape, expert_weights: ExpertWeights,
            W_gate: Optional[np.ndarray] = None,
            bias: Optional[np.ndarray] = None,
            logits: Optional[np.ndarray] = None,
            tokens: Optional[Sequence[int]] = None) -> dict:
    """Run the layer for all T tokens' routing and the requested tokens' output.

    expert_weights(e) returns (W1[e], W3[e], W2[e]); experts E .. E+S-1 are the
    shared ones.  Either W_gate (+ optional bias) or precomputed router logits
    must be given.  ``tokens`` limits which output rows are computed (routing,
    dispatch and statistics always cover all T tokens); rows not computed are
    NaN in ``out``.
    """
    T, d, E, k, S = shape.T, shape.d, shape.E, shape.k, shape.S
    x = np.asarray(x)
    if logits is None:
        logits = router_logits(x, W_gate, bias)
    logits = np.asarray(logits, dtype=np.float64)
    sel, margin = topk_select(logits, k)
    w = gate_weights(logits, sel, shape.gating, shape.renormalize)
    p = softmax_all(logits) if T > 0 else np.zeros((0, E))
    C = capacity(T, k, E, shape.capacity_factor)
    disp = dispatch_policy(sel, logits, E, C, shape.overflow)
    stats = routing_stats(disp["counts"], disp["kept"], p, T, k, E)

    want = np.zeros(T, dtype=bool)
    if tokens is None:
        want[:] = True
    else:
        want[np.asarray(list(tokens), dtype=np.int64)] = True
    out = np.full((T, d), np.nan)
    out[want] = 0.0

    # Routed experts: each expert runs once on its kept rows, in slot order.
    yrows = {}   # assignment a -> the output row of the expert that ran it
    for e in range(E):
        lo, hi = int(disp["offsets"][e]), int(disp["offsets"][e + 1])
        rows = [int(a) for a in disp["perm"][lo:hi] if want[int(a) // k]]
        if not rows:
            continue
        W1e, W3e, W2e = expert_weights(e)
        toks = [a // k for a in rows]
        Y = expert_ffn(np.asarray(x[toks], dtype=np.float64), W1e, W3e, W2e)
        for r, a in enumerate(rows):
            t, j = divmod(a, k)
            out[t] += w[t, j] * Y[r]
            yrows[a] = Y[r]

    # Shared experts: every token, gate 1.
    shared = None
    if S > 0:
        idx = np.nonzero(want)[0]
        shared = np.zeros((len(idx), d))
        for s in range(S):
            W1s, W3s, W2s = expert_weights(E + s)
            shared += expert_ffn(np.asarray(x[idx], dtype=np.float64),
                                 W1s, W3s, W2s)
        out[idx] += shared

    return dict(out=out, logits=logits, sel=sel, margin=margin, w=w, p=p,
                capacity=C, dispatch=disp, stats=stats, yrows=yrows)


# ---------------------------------------------------------------------------
# Router backward.  [Routing guide] "Plain explanation" paragraph 2: the
# router is trained together with the experts through the softmax, so a
# token's gradient reaches the scores of experts it did not pick (in the
# softmax-over-all order); paragraph 4: the auxiliary product E sum f_i P_i
# pushes the load back towards balance through P_i.  The selection, the
# capacity decisions and the counts f_i are piecewise constant and carry no
# gradient.
# ---------------------------------------------------------------------------
def router_backward(x: np.ndarray, W_gate: np.ndarray, fwd: dict,
                    shape: LayerShape, dout: np.ndarray,
                    aux_coef: float = 0.0,
                    tokens: Optional[Sequence[int]] = None,
                    entropy_coef: float = 0.0) -> dict:
    """Gradients of  L = sum(dout * out) + aux_coef * aux
    + entropy_coef * H_tok  with respect to the
    gate weights (dw [T, k]), the router scores (dlogits [T, E]), W_gate
    (dW_gate [d, E]), the bias (dbias [E]) and the router's share of dx
    ([T, d]; the experts' share is not part of this).  ``fwd`` is the result
    of ``forward`` for all T tokens.

      dw[t, j]   = dout[t] . y_{t,j} for an assignment some expert ran, else 0
      top-k then softmax (and renormalised softmax then top-k): the gates are a
      softmax over the k chosen scores, so for chosen c_i
          dl[t, c_i] = w_i (dw_i - sum_j w_j dw_j),   0 elsewhere;
      softmax over all experts, read at the chosen ones: w_j = p[t, c_j], so
          dl[t, i]  = p_i (G_i - sum_j w_j dw_j),   G_i = dw_j if i = c_j else 0,
      which is non-zero for every expert the token did not choose;
      aux = E sum_i f_i P_i with P_i = mean_t p[t, i] and f fixed:
          dl[t, m] += aux_coef (E / T) p[t, m] (f_m - sum_i f_i p[t, i]);
      H_tok = mean_t H_t, H_t = -sum_i p_ti ln p_ti (the router entropy that
      [Routing guide] "Plain explanation" paragraph 4 schedules, high early
      in training and lower later):
          dl[t, m] += entropy_coef (1 / T) (-p[t, m] (ln p[t, m] + H_t));
      scores l = x W_gate + b:  dW_gate = x^T dl, dbias = sum_t dl[t],
      dx = dl W_gate^T.
    ``tokens`` limits dw, dlogits and dx to those tokens (the others are NaN;
    ``forward`` must have computed their rows) and leaves out dW_gate and
    dbias, which need every token.
    """
    T, E, k = shape.T, shape.E, shape.k
    x64 = np.asarray(x, dtype=np.float64)
    W64 = np.asarray(W_gate, dtype=np.float64)
    g = np.asarray(dout, dtype=np.float64)
    sel, w, p = fwd["sel"], fwd["w"], fwd["p"]
    yrows = fwd["yrows"]
    todo = range(T) if tokens is None else sorted(set(int(t) for t in tokens))
    dw = np.zeros((T, k)) if tokens is None else np.full((T, k), np.nan)
    for t in todo:
        dw[t] = 0.0
        for j in range(k):
            a = t * k + j
            if a in yrows:
                dw[t, j] = float(np.dot(g[t], yrows[a]))
            elif fwd["dispatch"]["slot"][a] >= 0:
                raise ValueError("forward did not compute every kept row")
    dl = np.zeros((T, E)) if tokens is None else np.full((T, E), np.nan)
    softmax_over_chosen = (shape.gating == TOPK_THEN_SOFTMAX or shape.renormalize)
    for t in todo:
        dl[t] = 0.0
        s = float(np.dot(w[t], dw[t]))
        if softmax_over_chosen:
            for j in range(k):
                dl[t, sel[t, j]] = w[t, j] * (dw[t, j] - s)
        else:
            G = np.zeros(E)
            for j in range(k):
                G[sel[t, j]] = dw[t, j]
            dl[t] = p[t] * (G - s)
    if aux_coef != 0.0 and T > 0:
        f = fwd["dispatch"]["counts"].astype(np.float64) / (T * k)
        for t in todo:
            dl[t] += aux_coef * (E / T) * p[t] * (f - float(np.dot(f, p[t])))
    if entropy_coef != 0.0 and T > 0:
        for t in todo:
            pt = p[t]
            with np.errstate(divide="ignore", invalid="ignore"):
                lnp = np.where(pt > 0, np.log(pt), 0.0)
            H = -float(np.sum(pt * lnp))
            dl[t] += entropy_coef / T * (-pt * (lnp + H))
    if tokens is not None:
        dx = np.full((T, x64.shape[1]), np.nan)
        for t in todo:
            dx[t] = dl[t] @ W64.T
        return dict(dw=dw, dlogits=dl, dW_gate=None, dbias=None, dx=dx)
    return dict(dw=dw, dlogits=dl, dW_gate=x64.T @ dl, dbias=dl.sum(axis=0),
                dx=dl @ W64.T)


# ---------------------------------------------------------------------------
# Training-side quantities around the router.  [Routing guide] "Plain
# explanation" paragraph 4: the router's entropy is kept high early in
# training and lowered later; "Key insights" item 3 names the trend of the
# load-balancing loss among the quantities to watch.
# ---------------------------------------------------------------------------
def entropy_schedule(step: int, total_steps: int, high: float, low: float) -> float:
    """Weight of the mean router entropy in the loss at ``step``: ``high`` at
    step 0, falling in a straight line to ``low`` at step total_steps - 1,
    held at the ends outside that range.  The page gives only the direction
    (high early, lower later); the straight line is the plainest shape with
    it.  A run of one step uses ``low``."""
    if total_steps <= 1:
        return float(low)
    s = min(max(int(step), 0), int(total_steps) - 1)
    return float(high) + (float(low) - float(high)) * s / (int(total_steps) - 1)


def load_balance_trend(values: Sequence[float]) -> dict:
    """Trend of a series of load-balancing losses, one per training step:
    the least-squares slope of value against step number (per step) and the
    mean.  Written out as the normal equations of the straight-line fit:
    slope = sum((i - i_mean)(v_i - v_mean)) / sum((i - i_mean)^2)."""
    n = len(values)
    if n < 2:
        raise ValueError("a trend needs at least two values")
    v = [float(a) for a in values]
    i_mean = (n - 1) / 2.0
    v_mean = sum(v) / n
    num = sum((i - i_mean) * (v[i] - v_mean) for i in range(n))
    den = sum((i - i_mean) ** 2 for i in range(n))
    return dict(slope=num / den, mean=v_mean, last=v[-1], n=n)


# ---------------------------------------------------------------------------
# Brute-force top-k, used only to pin topk_select on tiny inputs.
# ---------------------------------------------------------------------------
def brute_topk_set(row: Sequence[float], k: int) -> tuple:
    """Among all k-subsets of experts, the one with the largest exact sum of
    logits; ties between subsets go to the lexicographically smallest sorted
    index tuple.  Sums are exact rationals, so -0.0 and +0.0 are equal."""
    from itertools import combinations
    vals = [Fraction(float(v)) for v in row]
    best, best_sum = None, None
    for combo in combinations(range(len(vals)), k):
        s = sum(vals[i] for i in combo)
        if best is None or s > best_sum or (s == best_sum and combo < best):
            best, best_sum = combo, s
    return best
