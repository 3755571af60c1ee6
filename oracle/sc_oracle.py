"""Plain float64 CPU oracle for the score-centering (SC) correction.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it, to check and to time the HIP
library.  It shares no code, table or constant generator with the HIP path.

Source of the method: "Score Centering" example page of Agent Lightning
(microsoft.github.io/agent-lightning, section "Score Centering").  That section
states, for one generated position:

* the rollout records the top-K behaviour probabilities q over an id set H from
  the sampling call, plus the sampled token a and its log-probability
  separately; the recorded q may sum to less than one and a may lie outside H;
* the trainer scores its own policy p over the whole vocabulary at the rollout
  temperature and gathers p at H and at a;
* with P_H = sum_H p_v, Q_H = sum_H q_v and
  rho = max(1 - Q_H, 1e-6) / max(1 - P_H, 1e-6), the token loss is
  -sg(A) * [log p_a - sum_H sg(q_v - rho p_v) log p_v];
* the unrecorded behaviour tail is taken to be proportional to p;
* the objective is unclipped, reduced over all generated tokens of the step,
  with padding masked; group standard-deviation normalisation gives A
  (same page, "Training" section);
* rollout_corr/k3_kl is the masked mean of exp(d) - 1 - d with
  d = train logprob - rollout logprob of the sampled token.

Readings taken where the page is silent (each is listed in the design notes):

* p is the trainer policy and q the recorded behaviour probabilities (the
  gradient flows through log p_a; the tail follows the shape of the policy
  being trained).
* 1 - P_H is evaluated as the direct off-head sum tau = sum_{v not in H} p_v,
  equal in exact arithmetic and free of cancellation.
* The behaviour estimate is mu_hat_v = q_k on H and rho * p_v off H.
* The centered score is the exact gradient of the bracket of the loss with
  respect to the tempered logits u = z / T:
  g = e_a - mu_hat - (1 - S) p, with S = sum_v mu_hat_v = Q_H + rho * tau.
  It equals e_a - mu_hat whenever S = 1 (no clamp binds).
* dLogits (gradient of the step loss sum_i loss_i / N_valid with respect to the
  raw logits z) is -A / (T * N_valid) * g.
* The correction is mu_hat - p.  TV is 1/2 sum_v |mu_hat_v - p_v| and KL is
  KL(mu_hat || p) = sum_v mu_hat_v log(mu_hat_v / p_v), over the full
  vocabulary, with 0 log 0 = 0.
* The argmax is taken on the raw logits; ties go to the lowest index.
* Data errors (id outside [0, V), duplicate id, sampled id outside [0, V),
  a NaN or +inf logit, a -inf logit at a recorded or sampled id) make every
  float output of the row NaN and its integer outputs -1.

Group normalisation (same page, "Training" section: advantages normalised by
the group's standard deviation; Agent Lightning v1.0.3 release note, section 4: rewards are not
rounded to bf16 first and the denominator must not overflow): rewards are
widened to float64; mode 0 divides by the unbiased standard deviation plus eps,
mode 1 by the population standard deviation plus eps, mode 2 only subtracts the
mean (the paper's mean-only setup the release note mentions).

bf16 rounding: round to nearest, ties to even (lecture notes "RL systems for
agents", section 4, where the cast is described).

LM head: the trainer's logits are the final hidden states times the
vocabulary projection, z = X W^T (one row of W per vocabulary id); the fused
LM-head path computes the same statistics from X and W without storing z.
"""
from __future__ import annotations

import math

import numpy as np

# Clamp constant printed in the rho definition (Score Centering section).
CLAMP = 1e-6

# Data-error bits; same meaning as the library's device status bits.
DEV_BAD_ID = 1
DEV_DUP_ID = 2
DEV_BAD_SAMPLED = 4
DEV_NONFINITE = 8
DEV_BAD_RESP = 16

# Importance-weighting modes (Score Centering page, SC settings table:
# is_mode none / tis / mis with tis_max 2.0 and the MIS interval [0.5, 5.0]).
IS_NONE = 0
IS_TIS = 1
IS_MIS = 2

# Row output modes for the full-vocabulary row.
MODE_DLOGITS = 0      # -A / (T * N_valid) * g
MODE_SCORE = 1        # g, the centered score
MODE_CORRECTION = 2   # mu_hat - p


def trainer_log_softmax(z, temperature):
    """log p over the full vocabulary at the rollout temperature.

    Score Centering page, section "Score Centering": the trainer evaluates
    its policy on every vocabulary id, at the temperature the rollout used.
    Returns (log p, lse) with lse = logsumexp(z / T) in float64.
    """
    u = np.asarray(z, dtype=np.float64) / float(temperature)
    m = np.max(u)
    s = np.sum(np.exp(u - m))
    lse = m + math.log(s)
    return u - lse, lse


def _row_flags(z, head_ids, sampled):
    """Data-error bits of one row (see the module docstring)."""
    V = z.shape[0]
    flags = 0
    ids = np.asarray(head_ids, dtype=np.int64)
    in_range = (ids >= 0) & (ids < V)
    if not np.all(in_range):
        flags |= DEV_BAD_ID
    good = ids[in_range]
    if np.unique(good).size != good.size:
        flags |= DEV_DUP_ID
    a_ok = 0 <= int(sampled) < V
    if not a_ok:
        flags |= DEV_BAD_SAMPLED
    if np.any(np.isnan(z)) or np.any(np.isposinf(z)):
        flags |= DEV_NONFINITE
    elif np.all(np.isneginf(z)):
        flags |= DEV_NONFINITE
    else:
        if np.any(np.isneginf(z[good])):
            flags |= DEV_NONFINITE
        if a_ok and np.isneginf(z[int(sampled)]):
            flags |= DEV_NONFINITE
    return flags


def is_weight(w, is_mode, lo, hi):
    """Stop-gradient weight of one token from its ratio w = p(a) / mu(a).

    Truncated IS replaces w by min(w, w_max) (lecture notes "RL systems for
    agents", section 1, where the truncated weight is defined); masked IS keeps
    the token, weighted by w, only when lo <= w <= hi and drops it otherwise
    (reading of the masked-IS setting with its acceptance interval,
    Score Centering page, SC settings).
    """
    if is_mode == IS_NONE:
        return 1.0
    if is_mode == IS_TIS:
        return min(w, hi)
    if is_mode == IS_MIS:
        return w if lo <= w <= hi else 0.0
    raise ValueError("is_mode")


def sc_row(z, temperature, head_ids, head_probs, sampled, rollout_logp=None,
           advantage=1.0, n_valid=1, row_mode=MODE_DLOGITS, is_mode=IS_NONE,
           is_lo=0.5, is_hi=None, centering=True):
    """All per-position SC outputs of one valid row, by definition, in float64.

    Arguments: z (V,) logits (any float dtype, widened exactly), temperature T,
    head_ids (K,) recorded ids H, head_probs (K,) recorded probabilities q,
    sampled id a, rollout_logp = log mu(a) recorded by the rollout (or None),
    advantage A of the row's response, n_valid = number of valid positions of
    the whole step, row_mode selecting the full-vocabulary row to return,
    is_mode / is_lo / is_hi the importance weighting of the token (needs
    rollout_logp), centering=False dropping the centering term (the grpo_mis
    ablation of the SC settings table, which turns centering off).

    Returns a dict; see the keys at the end.
    """
    z = np.asarray(z, dtype=np.float64)
    V = z.shape[0]
    ids = np.asarray(head_ids, dtype=np.int64)
    q = np.asarray(head_probs, dtype=np.float64)
    K = ids.shape[0]
    a = int(sampled)
    T = float(temperature)

    flags = _row_flags(z, ids, a)
    if flags:
        nan = float("nan")
        return dict(flags=flags, lse=nan, logp_a=nan, argmax=-1, a_slot=-1,
                    head_logp=np.full(K, nan), P_H=nan, Q_H=nan, tau=nan,
                    rho=nan, coef=np.full(K, nan), S=nan, loss=nan, tv=nan,
                    kl=nan, k3=nan, entropy=nan, w=nan, weight=nan,
                    rev_kl=nan, row=np.full(V, nan))

    # Trainer softmax at the rollout temperature; gather at H and at a.
    logp, lse = trainer_log_softmax(z, T)
    p = np.exp(logp)
    argmax = int(np.argmax(z))          # numpy returns the first maximum
    logp_a = logp[a]
    head_logp = logp[ids]
    p_H = p[ids]
    hits = np.nonzero(ids == a)[0]
    a_slot = int(hits[0]) if hits.size else -1

    # Masses: P_H, Q_H and the off-head trainer mass tau (= 1 - P_H exactly).
    in_H = np.zeros(V, dtype=bool)
    in_H[ids] = True
    P_H = float(np.sum(p_H))
    Q_H = float(np.sum(q))
    tau = float(np.sum(p[~in_H]))

    # rho with both clamps, as printed.
    rho = max(1.0 - Q_H, CLAMP) / max(tau, CLAMP)

    # Importance ratio of the sampled token and its stop-gradient weight.
    if rollout_logp is None:
        if is_mode != IS_NONE:
            raise ValueError("importance weighting needs rollout_logp")
        w = float("nan")
    else:
        w = math.exp(logp_a - float(rollout_logp))
    if is_hi is None:
        # settings-table defaults: TIS cap 2.0, MIS interval [0.5, 5.0]
        is_hi = 5.0 if is_mode == IS_MIS else 2.0
    weight = is_weight(w, is_mode, is_lo, is_hi)

    # Stop-gradient coefficients and the token loss.
    coef = q - rho * p_H
    centered = float(np.sum(coef * head_logp)) if centering else 0.0
    loss = -float(advantage) * weight * (logp_a - centered)

    # Behaviour estimate mu_hat: recorded head, tail proportional to p.
    mu_hat = rho * p
    mu_hat[ids] = q
    S = float(np.sum(mu_hat))

    # Centered score: gradient of the bracket with respect to u = z / T
    # (without centering: the plain score e_a - p), times the weight.
    g = (-mu_hat - (1.0 - S) * p) if centering else -p.copy()
    g[a] += 1.0
    g *= weight

    if row_mode == MODE_DLOGITS:
        row = (-float(advantage) / (T * float(n_valid))) * g
    elif row_mode == MODE_SCORE:
        row = g
    elif row_mode == MODE_CORRECTION:
        row = mu_hat - p
    else:
        raise ValueError("row_mode")

    # Diagnostics over the full vocabulary.
    tv = 0.5 * float(np.sum(np.abs(mu_hat - p)))
    pos = mu_hat > 0
    kl = float(np.sum(mu_hat[pos] * (np.log(mu_hat[pos]) - logp[pos])))
    if rollout_logp is None:
        k3 = float("nan")
    else:
        d = logp_a - float(rollout_logp)
        k3 = math.expm1(d) - d
    # Extra per-position signals (lecture notes, section 7, list of debugging
    # signals: entropy and the largest importance weight): the trainer
    # entropy -sum p log p and the reverse divergence KL(p || mu_hat).
    ppos = p > 0
    entropy = -float(np.sum(p[ppos] * logp[ppos]))
    if np.any(ppos & (mu_hat <= 0)):
        rev_kl = float("inf")
    else:
        rev_kl = float(np.sum(p[ppos] * (logp[ppos] - np.log(mu_hat[ppos]))))

    return dict(flags=0, lse=lse, logp_a=logp_a, argmax=argmax, a_slot=a_slot,
                head_logp=head_logp, P_H=P_H, Q_H=Q_H, tau=tau, rho=rho,
                coef=coef, S=S, loss=loss, tv=tv, kl=kl, k3=k3,
                entropy=entropy, w=w, weight=weight, rev_kl=rev_kl, row=row)


def sc_center_row(logp_a, tau, head_logp, head_probs, rollout_logp=None,
                  advantage=1.0, is_mode=IS_NONE, is_lo=0.5, is_hi=None,
                  centering=True):
    """The centering step of one valid row from the statistics it is handed,
    in float64: what a second call computes when it has the first call's
    log p(a), tail mass tau and log p at H but not the logits.

    Same definitions as sc_row (Score Centering page, section "Score
    Centering": rho with both 1e-6 clamps, c = q - rho p on H, the token loss;
    the tail of mu_hat is rho p), with every sum over the tail taken in closed
    form from tau: S = Q_H + rho tau, the tail's share of TV is
    |rho - 1| tau / 2, of KL(mu_hat || p) rho tau log rho and of KL(p ||
    mu_hat) -tau log rho.  p at H is exp(head_logp).

    Returns dict(P_H, Q_H, rho, S, coef, loss, tv, kl, rev_kl, k3, w, weight).
    """
    lp = np.asarray(head_logp, dtype=np.float64)
    q = np.asarray(head_probs, dtype=np.float64)
    logp_a = float(logp_a)
    tau = float(tau)
    p_H = np.exp(lp)
    P_H = float(np.sum(p_H))
    Q_H = float(np.sum(q))
    rho = max(1.0 - Q_H, CLAMP) / max(tau, CLAMP)

    if rollout_logp is None:
        if is_mode != IS_NONE:
            raise ValueError("importance weighting needs rollout_logp")
        w = float("nan")
        k3 = float("nan")
    else:
        d = logp_a - float(rollout_logp)
        w = math.exp(d)
        k3 = math.expm1(d) - d
    if is_hi is None:
        is_hi = 5.0 if is_mode == IS_MIS else 2.0
    weight = is_weight(w, is_mode, is_lo, is_hi)

    coef = q - rho * p_H
    centered = float(np.sum(coef * lp)) if centering else 0.0
    loss = -float(advantage) * weight * (logp_a - centered)
    S = Q_H + rho * tau

    log_rho = math.log(rho)
    tv = 0.5 * (float(np.sum(np.abs(q - p_H))) + abs(rho - 1.0) * tau)
    qpos = q > 0
    kl = float(np.sum(q[qpos] * (np.log(q[qpos]) - lp[qpos]))) + rho * tau * log_rho
    ppos = p_H > 0
    if np.any(ppos & ~qpos):
        rev_kl = float("inf")
    else:
        rev_kl = float(np.sum(p_H[ppos] * (lp[ppos] - np.log(q[ppos])))) - tau * log_rho
    return dict(P_H=P_H, Q_H=Q_H, rho=rho, S=S, coef=coef, loss=loss, tv=tv,
                kl=kl, rev_kl=rev_kl, k3=k3, w=w, weight=weight)


def masked_row(V, K):
    """Outputs of a padding row: nothing read, zero loss and gradient."""
    return dict(flags=0, lse=0.0, logp_a=0.0, argmax=-1, a_slot=-1,
                head_logp=np.zeros(K), P_H=0.0, Q_H=0.0, tau=0.0, rho=0.0,
                coef=np.zeros(K), S=0.0, loss=0.0, tv=0.0, kl=0.0, k3=0.0,
                entropy=0.0, w=0.0, weight=0.0, rev_kl=0.0, row=np.zeros(V))


def group_norm(rewards, group_size, mode=0, eps=1e-6):
    """Rollout-level advantages by group normalisation, in float64.

    Groups are consecutive runs of group_size responses.  mode 0: unbiased
    standard deviation, mode 1: population standard deviation, mode 2: mean
    only.  A group of one response gets advantage 0.
    """
    r = np.asarray(rewards, dtype=np.float64).reshape(-1, group_size)
    out = np.zeros_like(r)
    G = group_size
    for j in range(r.shape[0]):
        mean = sum(float(x) for x in r[j]) / G
        dev = [float(x) - mean for x in r[j]]
        if mode == 2:
            out[j] = dev
            continue
        if G == 1:
            out[j] = 0.0
            continue
        ss = sum(d * d for d in dev)
        std = math.sqrt(ss / (G - 1 if mode == 0 else G))
        out[j] = [d / (std + eps) for d in dev]
    return out.reshape(-1)


BATCH_KEYS = ("loss", "k3", "tv", "kl", "Q_H", "P_H", "entropy", "rev_kl")


def batch_sums(rows, n_valid):
    """Step-level reductions over valid rows (global generated-token mean).

    rows: iterable of sc_row() dicts of the valid rows.  Returns the sums and
    the means over n_valid, in float64, of BATCH_KEYS, plus the largest
    importance ratio w of the step under the key "max_w".
    """
    sums = {k: 0.0 for k in BATCH_KEYS}
    max_w = float("-inf")
    for r in rows:
        for k in BATCH_KEYS:
            sums[k] += float(r[k])
        max_w = max(max_w, float(r["w"]))
    means = {k: sums[k] / float(n_valid) for k in BATCH_KEYS}
    means["max_w"] = max_w
    return sums, means


def bf16_rne(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bf16 keeps 8 significant bits and float32's exponent range (subnormal
    spacing 2^-133).  Values beyond the largest finite bf16 after rounding
    become infinities.  Returned as float64.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    m, e = np.frexp(np.abs(xf))                 # |x| = m * 2^e, m in [0.5, 1)
    ulp_exp = np.maximum(e - 8, -133)           # spacing of 8 significant bits
    scaled = np.ldexp(np.abs(xf), -ulp_exp)     # exact (power-of-two scaling)
    r = np.rint(scaled)                         # round half to even
    mag = np.ldexp(r, ulp_exp)
    max_bf16 = float(np.ldexp(255.0, 127 - 7))  # (2 - 2^-7) * 2^127
    mag = np.where(mag > max_bf16, np.inf, mag)
    out[fin] = np.sign(xf) * mag
    return out


def lmhead_logits(hidden, weight):
    """Trainer logits z = X W^T of the LM head, in float64.

    hidden: (n, d) final hidden states, weight: (V, d) vocabulary projection
    with one row per id (both given as exactly widened bf16 values).  The
    Score Centering page's trainer scores the policy from these logits over
    the full vocabulary (section "Score Centering"); the product is the
    library matmul in float64, whose error on bf16 inputs (d <= 8192) is far
    below any fp32 tolerance.
    """
    X = np.asarray(hidden, dtype=np.float64)
    W = np.asarray(weight, dtype=np.float64)
    if X.ndim != 2 or W.ndim != 2 or X.shape[1] != W.shape[1]:
        raise ValueError("hidden (n, d) and weight (V, d) must agree on d")
    return X @ W.T


def record_topk(z, temperature, k, sampled=None):
    """The rollout engine's record of one position (rollout side of the method).

    Score Centering page, section "Score Centering": each generated position
    records the top K behaviour probabilities of the sampling call (their
    original normalisation kept, so they may sum below one) and, separately,
    the log-probability of the token actually sampled.

    z: (V,) rollout logits, temperature T, k recorded candidates, sampled id
    (or None).  The candidates are the k largest logits, ties to the lower
    id, listed in that order (probability descending, since softmax at T > 0
    keeps the order of the logits).  Returns dict(flags, head_ids, head_probs,
    sampled_logp) with head_probs = softmax(z / T) at head_ids in float64.
    A NaN or +inf logit, an all -inf row, a sampled id outside [0, V) or a
    sampled id at a -inf logit is a data error: ids -1, floats NaN.
    """
    z = np.asarray(z, dtype=np.float64)
    V = z.shape[0]
    if not 1 <= k <= V:
        raise ValueError("k")
    flags = 0
    if np.any(np.isnan(z)) or np.any(np.isposinf(z)) or np.all(np.isneginf(z)):
        flags |= DEV_NONFINITE
    if sampled is not None:
        if not 0 <= int(sampled) < V:
            flags |= DEV_BAD_SAMPLED
        elif np.isneginf(z[int(sampled)]):
            flags |= DEV_NONFINITE
    if flags:
        return dict(flags=flags, head_ids=np.full(k, -1), head_probs=np.full(k, np.nan),
                    sampled_logp=float("nan"))
    logp, _ = trainer_log_softmax(z, temperature)
    # lexsort: last key is the primary one (logit descending), then id ascending
    order = np.lexsort((np.arange(V), -z))[:k]
    return dict(flags=0, head_ids=order.astype(np.int64),
                head_probs=np.exp(logp[order]),
                sampled_logp=float(logp[int(sampled)]) if sampled is not None else float("nan"))


def lmhead_backward(hidden, weight, dlogits):
    """Gradients of the step loss through the LM head z = X W^T, in float64.

    dlogits: (n, V) gradient of the step loss with respect to the logits (the
    dLogits rows of sc_row, zero on padding rows).  By the chain rule through
    z = X W^T: dHidden = dZ W (n, d) and dW = dZ^T X (V, d).
    """
    X = np.asarray(hidden, dtype=np.float64)
    W = np.asarray(weight, dtype=np.float64)
    G = np.asarray(dlogits, dtype=np.float64)
    if G.shape != (X.shape[0], W.shape[0]) or X.shape[1] != W.shape[1]:
        raise ValueError("shapes")
    return G @ W, G.T @ X
