"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test fixes the oracle to something independent of its own code: values
derived by hand in closed form, autograd of the printed loss, brute force over
tiny vocabularies, library routines in special cases, invariants, and the
numbers printed on the pages (bf16 facts, the 1.0 vs 1.001 reward case).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import sc_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

LN = math.log
P4 = np.array([0.1, 0.2, 0.3, 0.4])
Z4 = np.log(np.array([1.0, 2.0, 3.0, 4.0]))   # softmax(Z4) = P4, lse = ln 10


# --------------------------------------------------------------------------
# Hand-derived cases (V = 4, p = [0.1, 0.2, 0.3, 0.4]).  Derivations follow
# the Score Centering section: P_H, Q_H, rho with clamps, c = q - rho p,
# loss = -A [log p_a - sum_H c log p], tail proportional to p.
# --------------------------------------------------------------------------
def _close(a, b, tol=1e-12):
    np.testing.assert_allclose(np.asarray(a, float), np.asarray(b, float),
                               rtol=0, atol=tol)


def test_hand_case_rho_one():
    # H = [3, 1], q = [0.5, 0.1], a = 2 (outside H).
    # P_H = 0.4 + 0.2 = 0.6, Q_H = 0.6, tau = 0.4, rho = 0.4 / 0.4 = 1.
    # c = [0.5 - 0.4, 0.1 - 0.2] = [0.1, -0.1];  mu_hat = [0.1, 0.1, 0.3, 0.5].
    # loss = -[ln .3 - (0.1 ln .4 - 0.1 ln .2)] = -ln .3 + 0.1 ln 2.
    # g = e_2 - mu_hat = [-0.1, -0.1, 0.7, -0.5];  dlogits(A=1,T=1,N=1) = -g.
    # TV = (0.1 + 0.1) / 2 = 0.1;  KL = 0.5 ln(0.5/0.4) + 0.1 ln(0.1/0.2).
    r = O.sc_row(Z4, 1.0, [3, 1], [0.5, 0.1], 2, rollout_logp=LN(0.15))
    _close(r["lse"], LN(10.0))
    _close(r["logp_a"], LN(0.3))
    _close(r["head_logp"], [LN(0.4), LN(0.2)])
    assert r["argmax"] == 3 and r["a_slot"] == -1
    _close([r["P_H"], r["Q_H"], r["tau"], r["rho"], r["S"]],
           [0.6, 0.6, 0.4, 1.0, 1.0])
    _close(r["coef"], [0.1, -0.1])
    _close(r["loss"], -LN(0.3) + 0.1 * LN(2.0))
    _close(r["row"], [0.1, 0.1, -0.7, 0.5])
    _close(r["tv"], 0.1)
    _close(r["kl"], 0.5 * LN(1.25) - 0.1 * LN(2.0))
    # K3 with d = ln .3 - ln .15 = ln 2:  e^d - 1 - d = 1 - ln 2.
    _close(r["k3"], 1.0 - LN(2.0))
    corr = O.sc_row(Z4, 1.0, [3, 1], [0.5, 0.1], 2,
                    row_mode=O.MODE_CORRECTION)["row"]
    _close(corr, [0.0, -0.1, 0.0, 0.1])


def test_hand_case_rho_half():
    # q = [0.6, 0.2]: Q_H = 0.8, rho = 0.2 / 0.4 = 0.5,
    # c = [0.6 - 0.2, 0.2 - 0.1] = [0.4, 0.1], mu_hat = [.05, .2, .15, .6].
    # loss = -[ln .3 - 0.4 ln .4 - 0.1 ln .2];  g = [-.05, -.2, .85, -.6].
    # TV = (0.2 + 0 + |0.5 - 1| * 0.4) / 2 = 0.2;
    # KL = 0.6 ln 1.5 + 0.2 ln 1 + 0.05 ln 0.5 + 0.15 ln 0.5.
    r = O.sc_row(Z4, 1.0, [3, 1], [0.6, 0.2], 2, row_mode=O.MODE_SCORE)
    _close(r["rho"], 0.5)
    _close(r["coef"], [0.4, 0.1])
    _close(r["loss"], -(LN(0.3) - 0.4 * LN(0.4) - 0.1 * LN(0.2)))
    _close(r["row"], [-0.05, -0.2, 0.85, -0.6])
    _close(r["tv"], 0.2)
    _close(r["kl"], 0.6 * LN(1.5) - 0.2 * LN(2.0))


def test_hand_case_sampled_in_head():
    # a = 1 = H[1]: a_slot = 1, logp_a = ln .2,
    # loss = -[ln .2 - 0.1 ln .4 + 0.1 ln .2];  g = e_1 - [.1, .1, .3, .5].
    r = O.sc_row(Z4, 1.0, [3, 1], [0.5, 0.1], 1, row_mode=O.MODE_SCORE)
    assert r["a_slot"] == 1
    _close(r["loss"], -(LN(0.2) - 0.1 * LN(0.4) + 0.1 * LN(0.2)))
    _close(r["row"], [-0.1, 0.9, -0.3, -0.5])


def test_hand_case_numerator_clamp():
    # q = [0.7, 0.3] sums to 1: max(1 - Q_H, 1e-6) = 1e-6, tau = 0.4,
    # rho = 2.5e-6, S = Q_H + rho tau = 1 + 1e-6.
    # g = e_a - mu_hat - (1 - S) p = e_2 - [2.5e-7, .3, 7.5e-7, .7] + 1e-6 p.
    r = O.sc_row(Z4, 1.0, [3, 1], [0.7, 0.3], 2, row_mode=O.MODE_SCORE)
    _close(r["rho"], 2.5e-6, 1e-18)
    _close(r["S"], 1.0 + 1e-6, 1e-15)
    _close(r["coef"], [0.7 - 1e-6, 0.3 - 5e-7], 1e-15)
    _close(r["row"], [-2.5e-7 + 1e-7, -0.3 + 2e-7, 1 - 7.5e-7 + 3e-7,
                      -0.7 + 4e-7], 1e-15)


def test_hand_case_full_head_matching():
    # K = V with q = p: 1 - Q_H = 0 and tau = 0, both clamp to 1e-6, rho = 1,
    # c = 0, mu_hat = p, correction 0, g = e_a - p, TV = KL = 0.
    r = O.sc_row(Z4, 1.0, [0, 1, 2, 3], P4, 0, row_mode=O.MODE_SCORE)
    _close(r["rho"], 1.0, 1e-9)
    _close(r["coef"], np.zeros(4), 1e-15)
    _close(r["row"], [0.9, -0.2, -0.3, -0.4], 1e-15)
    _close([r["tv"], r["kl"]], [0.0, 0.0], 1e-15)
    corr = O.sc_row(Z4, 1.0, [0, 1, 2, 3], P4, 0,
                    row_mode=O.MODE_CORRECTION)["row"]
    _close(corr, np.zeros(4), 1e-15)


def test_hand_case_temperature_and_scaling():
    # z = 0.5 ln k at T = 0.5 gives the same p.  With A = -1, N_valid = 4:
    # dlogits = -A / (T N) g = 0.5 g, g as in the rho = 0.5 case; loss flips.
    r = O.sc_row(0.5 * Z4, 0.5, [3, 1], [0.6, 0.2], 2, advantage=-1.0,
                 n_valid=4)
    _close(r["lse"], LN(10.0))
    _close(r["loss"], LN(0.3) - 0.4 * LN(0.4) - 0.1 * LN(0.2))
    _close(r["row"], 0.5 * np.array([-0.05, -0.2, 0.85, -0.6]))


# --------------------------------------------------------------------------
# Autograd of the printed token loss (torch, float64)
# --------------------------------------------------------------------------
def _printed_loss(z, T, ids, q, a, A, n_valid):
    """-sg(A) [log p_a - sum_H sg(q - rho p) log p] / N_valid at temperature T,
    written from the Score Centering section with detach() as sg."""
    logp = torch.log_softmax(z / T, dim=0)
    p = logp.exp()
    P_H = p[ids].sum()
    Q_H = q.sum()
    rho = torch.clamp(1 - Q_H, min=1e-6) / torch.clamp(1 - P_H, min=1e-6)
    c = (q - rho * p[ids]).detach()
    return -A * (logp[a] - (c * logp[ids]).sum()) / n_valid


def _rand_case(rng, V, K, clamp=None):
    z = rng.normal(0, 2.0, V)
    ids = rng.choice(V, K, replace=False)
    p = np.exp(z - z.max()); p /= p.sum()
    if clamp == "tail":          # trainer tail below 1e-6, recorded head short
        z = rng.normal(0, 1.0, V)
        z[ids] += 30.0
        q = rng.dirichlet(np.ones(K)) * 0.9
    elif clamp == "head":        # recorded head sums to >= 1
        q = rng.dirichlet(np.ones(K)) * (1 + 1e-7)
    else:
        q = rng.dirichlet(np.ones(K)) * rng.uniform(0.3, 0.99)
    a = int(rng.integers(V))
    return z, ids, q, a


@pytest.mark.parametrize("T", [1.0, 0.7])
@pytest.mark.parametrize("clamp", [None, "tail", "head"])
def test_dlogits_equal_autograd_of_printed_loss(T, clamp):
    rng = np.random.default_rng(123)
    for V in (8, 16, 32):
        for trial in range(20):
            K = int(rng.integers(1, V))
            z, ids, q, a = _rand_case(rng, V, K, clamp)
            A = float(rng.normal())
            n_valid = int(rng.integers(1, 50))
            zt = torch.tensor(z, dtype=torch.float64, requires_grad=True)
            loss = _printed_loss(zt, T, torch.tensor(ids), torch.tensor(q), a,
                                 A, n_valid)
            loss.backward()
            r = O.sc_row(z, T, ids, q, a, advantage=A, n_valid=n_valid)
            np.testing.assert_allclose(r["row"], zt.grad.numpy(), rtol=1e-9,
                                       atol=1e-11)
            np.testing.assert_allclose(r["loss"] / n_valid, loss.item(),
                                       rtol=1e-10, atol=1e-10)


def test_clamp_reading_differs_from_plain_centering():
    # When tau < 1e-6 and 1 - Q_H >> 1e-6, S != 1 and the exact gradient
    # e_a - mu_hat - (1 - S) p differs from e_a - mu_hat by (1 - S) p.
    rng = np.random.default_rng(5)
    z, ids, q, a = _rand_case(rng, 16, 4, "tail")
    r = O.sc_row(z, 1.0, ids, q, a, row_mode=O.MODE_SCORE)
    assert r["tau"] < 1e-6 and r["S"] < 0.95
    logp, _ = O.trainer_log_softmax(z, 1.0)
    p = np.exp(logp)
    corr = O.sc_row(z, 1.0, ids, q, a, row_mode=O.MODE_CORRECTION)["row"]
    plain = np.eye(16)[a] - (corr + p)
    np.testing.assert_allclose(plain - r["row"], (1 - r["S"]) * p, atol=1e-12)
    assert np.abs(plain - r["row"]).max() > 0.01


# --------------------------------------------------------------------------
# Brute force: centering removes the mean update when the tail really is
# proportional to p (release note, section 1: "removes average update bias")
# --------------------------------------------------------------------------
def test_centering_identity_brute_force():
    rng = np.random.default_rng(7)
    for V in (4, 8, 16):
        for trial in range(50):
            K = int(rng.integers(1, V))
            z = rng.normal(0, 1.5, V)
            p = np.exp(z - z.max()); p /= p.sum()
            ids = rng.choice(V, K, replace=False)
            in_H = np.zeros(V, bool); in_H[ids] = True
            # a behaviour policy: arbitrary head mass, tail exactly prop. to p
            q = rng.dirichlet(np.ones(K)) * rng.uniform(0.2, 0.95)
            mu = np.zeros(V)
            mu[ids] = q
            mu[~in_H] = (1 - q.sum()) * p[~in_H] / p[~in_H].sum()
            assert abs(mu.sum() - 1) < 1e-12
            expected = np.zeros(V)
            for a in range(V):
                r = O.sc_row(z, 1.0, ids, q, a, row_mode=O.MODE_SCORE)
                expected += mu[a] * r["row"]
                corr = O.sc_row(z, 1.0, ids, q, a,
                                row_mode=O.MODE_CORRECTION)["row"]
                np.testing.assert_allclose(corr, mu - p, atol=1e-13)
            np.testing.assert_allclose(expected, 0.0, atol=1e-13)


# --------------------------------------------------------------------------
# Special cases that reduce to library routines
# --------------------------------------------------------------------------
def test_log_softmax_and_lse_match_torch():
    rng = np.random.default_rng(1)
    for T in (1.0, 0.7, 2.5):
        z = rng.normal(0, 3, 1000)
        logp, lse = O.trainer_log_softmax(z, T)
        zt = torch.tensor(z, dtype=torch.float64) / T
        np.testing.assert_allclose(logp, torch.log_softmax(zt, 0).numpy(),
                                   atol=1e-12)
        assert abs(lse - torch.logsumexp(zt, 0).item()) < 1e-12


def test_identical_distributions_give_cross_entropy_gradient():
    # q = p on H: rho = 1, mu_hat = p, correction 0 and the SC gradient is
    # A / N_valid times the cross-entropy gradient (torch autograd).
    rng = np.random.default_rng(2)
    V, K, T = 64, 10, 0.8
    for trial in range(10):
        z = rng.normal(0, 2, V)
        logp, _ = O.trainer_log_softmax(z, T)
        ids = rng.choice(V, K, replace=False)
        q = np.exp(logp[ids])
        a = int(rng.integers(V))
        A, n_valid = float(rng.normal()), 7
        r = O.sc_row(z, T, ids, q, a, advantage=A, n_valid=n_valid)
        assert abs(r["rho"] - 1) < 1e-12
        _close(r["coef"], np.zeros(K), 1e-13)
        zt = torch.tensor(z, dtype=torch.float64, requires_grad=True)
        torch.nn.functional.cross_entropy((zt / T)[None], torch.tensor([a])
                                          ).backward()
        np.testing.assert_allclose(r["row"], A / n_valid * zt.grad.numpy(),
                                   atol=1e-13)
        corr = O.sc_row(z, T, ids, q, a, row_mode=O.MODE_CORRECTION)["row"]
        _close(corr, np.zeros(V), 1e-13)
        assert r["tv"] < 1e-13 and abs(r["kl"]) < 1e-13


def test_argmax_lowest_index_on_ties():
    z = np.array([0.0, 3.0, -1.0, 3.0, 3.0, 2.0])
    r = O.sc_row(z, 1.0, [5], [0.1], 0)
    assert r["argmax"] == 1


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------
def test_invariants_random_rows():
    rng = np.random.default_rng(3)
    for trial in range(200):
        V = int(rng.integers(2, 300))
        K = int(rng.integers(1, V + 1))
        clamp = rng.choice([None, "tail", "head"])
        z, ids, q, a = _rand_case(rng, V, K, clamp)
        r = O.sc_row(z, 1.0, ids, q, a, row_mode=O.MODE_SCORE)
        logp, _ = O.trainer_log_softmax(z, 1.0)
        p = np.exp(logp)
        assert abs(r["P_H"] + r["tau"] - 1) < 1e-12
        assert abs(r["P_H"] - p[ids].sum()) < 1e-12
        # the gradient of any log-softmax loss sums to zero over the vocabulary
        assert abs(r["row"].sum()) < 1e-12
        # S = Q_H + rho tau, and S = 1 when no clamp binds
        assert abs(r["S"] - (r["Q_H"] + r["rho"] * r["tau"])) < 1e-12
        if 1 - r["Q_H"] >= 1e-6 and r["tau"] >= 1e-6:
            assert abs(r["S"] - 1) < 1e-12
        # TV in [0, 1] when S = 1; equals sum max(0, p - mu_hat) then
        # (lecture notes, exercise 2 and its solution)
        corr = O.sc_row(z, 1.0, ids, q, a, row_mode=O.MODE_CORRECTION)["row"]
        mu_hat = corr + p
        if abs(r["S"] - 1) < 1e-12:
            assert abs(r["tv"] - np.maximum(0, p - mu_hat).sum()) < 1e-12
        # closed forms of TV and KL(mu_hat || p): the tail is prop. to p
        in_H = np.zeros(V, bool); in_H[ids] = True
        tv_cf = 0.5 * (np.abs(q - p[ids]).sum() + abs(r["rho"] - 1) * r["tau"])
        qpos = q > 0
        kl_cf = (q[qpos] * (np.log(q[qpos]) - logp[ids][qpos])).sum()
        if r["rho"] * r["tau"] > 0:
            kl_cf += r["rho"] * r["tau"] * math.log(r["rho"])
        assert abs(r["tv"] - tv_cf) < 1e-12
        assert abs(r["kl"] - kl_cf) < 1e-10 * max(1, abs(kl_cf))


def test_k3_properties():
    # rollout_corr/k3_kl term exp(d) - 1 - d (Score Centering section):
    # >= 0, zero iff d = 0, e - 2 at d = 1, ~ d^2 / 2 for small d.
    z = np.log(np.array([1.0, 2.0, 3.0, 4.0]))
    for d in (-3.0, -0.5, 1e-4, 0.0, 1.0, 2.0):
        r = O.sc_row(z, 1.0, [3], [0.4], 2, rollout_logp=LN(0.3) - d)
        assert r["k3"] >= 0
        if d == 0:
            assert r["k3"] == 0
        if d == 1.0:
            _close(r["k3"], math.e - 2)
        if d == 1e-4:
            _close(r["k3"], d * d / 2, 1e-12)


# --------------------------------------------------------------------------
# Data errors and padding
# --------------------------------------------------------------------------
def test_data_error_flags():
    z = np.zeros(8)
    assert O.sc_row(z, 1.0, [1, 9], [.1, .1], 0)["flags"] == O.DEV_BAD_ID
    assert O.sc_row(z, 1.0, [1, 1], [.1, .1], 0)["flags"] == O.DEV_DUP_ID
    assert O.sc_row(z, 1.0, [1, 2], [.1, .1], 8)["flags"] == O.DEV_BAD_SAMPLED
    zn = z.copy(); zn[5] = np.nan
    r = O.sc_row(zn, 1.0, [1, 2], [.1, .1], 0)
    assert r["flags"] == O.DEV_NONFINITE and np.isnan(r["loss"])
    zi = z.copy(); zi[2] = -np.inf
    assert O.sc_row(zi, 1.0, [1, 2], [.1, .1], 0)["flags"] == O.DEV_NONFINITE
    # -inf outside H and a is a legal masked vocabulary entry (p = 0)
    r = O.sc_row(zi, 1.0, [1, 3], [.1, .1], 0)
    assert r["flags"] == 0 and np.isfinite(r["loss"]) and r["row"][2] == 0


# --------------------------------------------------------------------------
# Group normalisation
# --------------------------------------------------------------------------
def test_group_norm_hand_cases():
    # R = [1, 0, 0, 0]: mean 0.25, unbiased std sqrt(0.75 / 3) = 0.5.
    A = O.group_norm([1, 0, 0, 0], 4, mode=0, eps=0.0)
    _close(A, [1.5, -0.5, -0.5, -0.5])
    # population std sqrt(0.75 / 4) = sqrt(3) / 4: A_1 = 0.75 / (sqrt 3 / 4).
    A = O.group_norm([1, 0, 0, 0], 4, mode=1, eps=0.0)
    _close(A[0], math.sqrt(3.0))
    _close(O.group_norm([1, 0, 0, 0], 4, mode=2), [0.75, -.25, -.25, -.25])
    # zero-variance groups and single-response groups give exactly 0
    assert np.all(O.group_norm([0.3] * 8, 4) == 0)
    assert np.all(O.group_norm([1.0, 0.0, 5.0], 1) == 0)


def test_group_norm_matches_statistics_module():
    import statistics
    rng = np.random.default_rng(4)
    for G in (2, 4, 8):
        r = rng.random(G * 6).astype(np.float32)
        A = O.group_norm(r, G, mode=0, eps=1e-6)
        for j in range(6):
            g = [float(x) for x in r[j * G:(j + 1) * G]]
            m, s = statistics.fmean(g), statistics.stdev(g)
            _close(A[j * G:(j + 1) * G], [(x - m) / (s + 1e-6) for x in g],
                   1e-12)


def test_group_norm_keeps_fractional_rewards_and_large_values():
    # Release note, section 4: 1.0 and 1.001 stay distinct (no bf16 cast);
    # the normaliser must not overflow for large rewards.
    A = O.group_norm(np.array([1.0, 1.001, 1.0, 1.001], np.float32), 4)
    assert A[0] < 0 < A[1] and abs(A[0] + A[1]) < 1e-9
    big = np.array([1e30, -1e30, 3e29, 0.0], np.float32)
    A = O.group_norm(big, 4)
    assert np.all(np.isfinite(A)) and abs(A.sum()) < 1e-9


def test_batch_sums_global_token_mean():
    rows = [dict(loss=1.0, k3=0.1, tv=0.2, kl=0.3, Q_H=0.9, P_H=0.8, entropy=2.0,
                 rev_kl=0.1, w=1.5),
            dict(loss=3.0, k3=0.3, tv=0.4, kl=0.5, Q_H=0.7, P_H=0.6, entropy=4.0,
                 rev_kl=0.3, w=0.5)]
    sums, means = O.batch_sums(rows, 4)
    _close([sums["loss"], means["loss"], means["Q_H"], means["entropy"]],
           [4.0, 1.0, 0.4, 1.5])
    assert means["max_w"] == 1.5


# --------------------------------------------------------------------------
# Importance weighting (TIS / MIS) and centering off
# --------------------------------------------------------------------------
def test_tis_worked_example_from_the_lecture_notes():
    with open(os.path.join(GOLDEN, "tis_page_example.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        # a two-token vocabulary whose trainer probability of token 0 is pi
        z = np.log(np.array([c["pi"], 1.0 - c["pi"]]))
        r = O.sc_row(z, 1.0, [1], [0.1], 0, rollout_logp=math.log(c["mu"]),
                     is_mode=O.IS_TIS, is_hi=c["w_max"])
        _close(r["w"], c["w"], 1e-12)
        _close(r["weight"], c["weight"], 1e-12)
        _close(max(0.0, c["pi"] - c["w_max"] * c["mu"]) if c["w"] > c["w_max"] else 0.0,
               c["bias_coef"], 1e-12)


def _behaviour_and_trainer(rng, V):
    pi = rng.dirichlet(np.ones(V) * 0.7)
    mu = rng.dirichlet(np.ones(V) * 0.7)
    return pi, mu


def test_tis_bias_equals_the_exact_formula_by_brute_force():
    # E_pi[f] - E_mu[min(w, w_max) f] = sum_{w > w_max} (pi - w_max mu) f
    # (lecture notes, section 1), with the oracle's weight for every token.
    rng = np.random.default_rng(31)
    for trial in range(30):
        V = int(rng.integers(3, 12))
        pi, mu = _behaviour_and_trainer(rng, V)
        f = rng.normal(size=V)
        z = np.log(pi)
        wmax = float(rng.uniform(1.0, 3.0))
        weights = np.array([O.sc_row(z, 1.0, [0], [0.1], a, rollout_logp=math.log(mu[a]),
                                     is_mode=O.IS_TIS, is_hi=wmax)["weight"]
                            for a in range(V)])
        lhs = np.sum(pi * f) - np.sum(mu * weights * f)
        w = pi / mu
        rhs = np.sum(np.where(w > wmax, pi - wmax * mu, 0.0) * f)
        assert abs(lhs - rhs) < 1e-12


def test_mis_keeps_exactly_the_accepted_tokens():
    # With weight w inside [lo, hi] and 0 outside, E_mu[weight f] is the
    # trainer expectation restricted to accepted tokens.
    rng = np.random.default_rng(32)
    for trial in range(30):
        V = int(rng.integers(3, 12))
        pi, mu = _behaviour_and_trainer(rng, V)
        f = rng.normal(size=V)
        z = np.log(pi)
        weights = np.array([O.sc_row(z, 1.0, [0], [0.1], a, rollout_logp=math.log(mu[a]),
                                     is_mode=O.IS_MIS, is_lo=0.5, is_hi=5.0)["weight"]
                            for a in range(V)])
        w = pi / mu
        acc = (w >= 0.5) & (w <= 5.0)
        assert abs(np.sum(mu * weights * f) - np.sum(np.where(acc, pi, 0) * f)) < 1e-12


@pytest.mark.parametrize("mode", ["tis", "mis"])
def test_weighted_and_uncentered_gradients_match_autograd(mode):
    # loss = -sg(A) sg(weight) [log p_a - centering sum_H sg(c) log p]
    rng = np.random.default_rng(33)
    is_mode = O.IS_TIS if mode == "tis" else O.IS_MIS
    for V in (8, 16):
        for trial in range(15):
            K = int(rng.integers(1, V))
            z, ids, q, a = _rand_case(rng, V, K)
            rlp = float(np.log(rng.uniform(0.01, 0.9)))
            A, n_valid = float(rng.normal()), 5
            for centering in (True, False):
                r = O.sc_row(z, 1.0, ids, q, a, rollout_logp=rlp, advantage=A,
                             n_valid=n_valid, is_mode=is_mode, is_lo=0.5, is_hi=2.0,
                             centering=centering)
                zt = torch.tensor(z, dtype=torch.float64, requires_grad=True)
                logp = torch.log_softmax(zt, 0)
                p = logp.exp()
                w = math.exp(float(logp[a].detach()) - rlp)
                weight = min(w, 2.0) if mode == "tis" else (w if 0.5 <= w <= 2.0 else 0.0)
                rho = torch.clamp(1 - torch.tensor(q).sum(), min=1e-6) / torch.clamp(
                    1 - p[torch.tensor(ids)].sum(), min=1e-6)
                c = (torch.tensor(q) - rho * p[torch.tensor(ids)]).detach()
                bracket = logp[a] - (c * logp[torch.tensor(ids)]).sum() * centering
                (-A * weight * bracket / n_valid).backward()
                np.testing.assert_allclose(r["row"], zt.grad.numpy(), rtol=1e-9, atol=1e-11)
                _close(r["weight"], weight, 1e-12)


def test_centering_off_is_the_weighted_policy_gradient():
    # centering disabled: g = weight (e_a - p), the plain importance-weighted
    # score (the grpo_mis ablation).
    rng = np.random.default_rng(34)
    z, ids, q, a = _rand_case(rng, 20, 5)
    logp, _ = O.trainer_log_softmax(z, 1.0)
    rlp = float(logp[a]) - 0.3
    r = O.sc_row(z, 1.0, ids, q, a, rollout_logp=rlp, row_mode=O.MODE_SCORE,
                 is_mode=O.IS_MIS, is_lo=0.5, is_hi=5.0, centering=False)
    expect = math.exp(0.3) * (np.eye(20)[a] - np.exp(logp))
    np.testing.assert_allclose(r["row"], expect, atol=1e-13)


# --------------------------------------------------------------------------
# Entropy and reverse KL
# --------------------------------------------------------------------------
def test_entropy_matches_torch_distribution():
    rng = np.random.default_rng(35)
    for T in (1.0, 0.6):
        z = rng.normal(0, 3, 500)
        r = O.sc_row(z, T, [1, 2], [0.1, 0.1], 0)
        ref = torch.distributions.Categorical(logits=torch.tensor(z / T)).entropy().item()
        assert abs(r["entropy"] - ref) < 1e-10
    # uniform logits: entropy log V
    r = O.sc_row(np.zeros(64), 1.0, [1], [0.1], 0)
    _close(r["entropy"], math.log(64), 1e-12)


def test_reverse_kl_closed_form_and_special_cases():
    rng = np.random.default_rng(36)
    for trial in range(50):
        V = int(rng.integers(3, 200))
        K = int(rng.integers(1, V))
        z, ids, q, a = _rand_case(rng, V, K, rng.choice([None, "tail", "head"]))
        r = O.sc_row(z, 1.0, ids, q, a)
        logp, _ = O.trainer_log_softmax(z, 1.0)
        p_h = np.exp(logp[ids])
        # the tail of mu_hat is rho p, so its part of sum p log(p / mu_hat)
        # is -tau log rho
        cf = np.sum(p_h * (logp[ids] - np.log(q))) - r["tau"] * math.log(r["rho"])
        assert abs(r["rev_kl"] - cf) < 1e-9 * max(1, abs(cf))
        assert r["rev_kl"] >= -1e-12 or r["S"] != 1
    # identical distributions: zero
    logp, _ = O.trainer_log_softmax(Z4, 1.0)
    r = O.sc_row(Z4, 1.0, [3, 1], np.exp(logp[[3, 1]]), 2)
    assert abs(r["rev_kl"]) < 1e-13
    # a recorded id with q = 0 but p > 0 makes the reverse KL infinite
    r = O.sc_row(Z4, 1.0, [3, 1], [0.5, 0.0], 2)
    assert r["rev_kl"] == float("inf")


# --------------------------------------------------------------------------
# bf16 round-to-nearest-even
# --------------------------------------------------------------------------
def test_center_from_statistics_matches_the_full_row():
    """sc_center_row, fed the log p(a), tau and log p at H of a row, gives
    every centering output of sc_row on that row: the closed-form tail sums
    (S, TV, both KL directions) against sc_row's sums over the whole
    vocabulary, at the clamp corners, with masks, every weighting and
    centering off."""
    rng = np.random.default_rng(123)
    cases = 0
    for case in range(48):
        V, K = 300, 40
        z = rng.normal(0, 2, V)
        ids = rng.choice(V, K, replace=False)
        kind = case % 6
        if kind == 1:
            z[ids] += 20.0                                   # tau < 1e-6
        if kind == 3:
            mask = rng.random(V) < 0.3
            mask[ids] = False
            z[mask] = -np.inf
        q = rng.dirichlet(np.ones(K)) * (rng.uniform(0.3, 0.95) if kind != 2 else 1.0 + 2.0 ** -20)
        if kind == 4:
            q[3] = 0.0                                       # reverse KL infinite
        a = int(ids[5]) if case % 2 else int(rng.integers(0, V))
        while a != ids[5] and np.isneginf(z[a]):
            a = int(rng.integers(0, V))
        rlp = float(np.log(rng.uniform(0.05, 1.0)))
        wkw = [dict(), dict(is_mode=O.IS_TIS, is_hi=1.5), dict(is_mode=O.IS_MIS, is_lo=0.5, is_hi=3.0),
               dict(centering=False)][case % 4]
        T = (1.0, 0.7, 1.3)[case % 3]
        o = O.sc_row(z, T, ids, q, a, rollout_logp=rlp, advantage=-0.8, **wkw)
        c = O.sc_center_row(o["logp_a"], o["tau"], o["head_logp"], q, rollout_logp=rlp,
                            advantage=-0.8, **wkw)
        if kind == 1:
            assert o["tau"] < 1e-6 and o["rho"] > 1e4
        for key in ("P_H", "Q_H", "rho", "S", "coef", "loss", "tv", "kl", "k3", "w", "weight"):
            np.testing.assert_allclose(c[key], o[key], rtol=1e-11, atol=1e-13, err_msg=f"{case} {key}")
        if math.isinf(o["rev_kl"]):
            assert c["rev_kl"] == o["rev_kl"]
        else:
            np.testing.assert_allclose(c["rev_kl"], o["rev_kl"], rtol=1e-11, atol=1e-13)
        cases += 1
    assert cases == 48


def test_bf16_page_facts():
    with open(os.path.join(GOLDEN, "bf16_page_facts.json")) as f:
        facts = json.load(f)
    for fact in facts["facts"]:
        got = O.bf16_rne(fact["x"])
        if "expect" in fact:
            assert got == fact["expect"], fact["what"]
        else:
            assert got == O.bf16_rne(fact["same_as"]), fact["what"]
    for case in facts["step_counts"]:
        v = O.bf16_rne(case["start"])
        master, steps = case["start"], 0
        while O.bf16_rne(master) == v:
            master += case["step"]
            steps += 1
        assert steps == case["steps"], case["what"]


def test_bf16_matches_torch_rne_on_float32_values():
    rng = np.random.default_rng(9)
    x = np.concatenate([
        rng.normal(0, 1, 20000), rng.normal(0, 1e-30, 2000),
        np.ldexp(rng.normal(0, 1, 2000), -130),   # bf16 subnormal range
        [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3.3e38, 3.4e38, 0.0],
    ]).astype(np.float32)
    ref = torch.tensor(x).to(torch.bfloat16).double().numpy()
    got = O.bf16_rne(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    # ties go to the even neighbour
    assert O.bf16_rne(1 + 2 ** -8) == 1.0
    assert O.bf16_rne(1 + 3 * 2 ** -8) == 1 + 2 ** -6


# --------------------------------------------------------------------------
# Generator sanity (the inputs the oracle is fed look like the pages' record)
# --------------------------------------------------------------------------
def test_tiny_generator_shapes_and_record():
    from synthetic import tiny
    d = tiny(seed=0)
    n, V = d["logits"].shape
    assert (n, V) == (256, 4096) and d["head_ids"].shape == (256, 128)
    for i in range(0, 256, 37):
        assert len(set(d["head_ids"][i])) == 128
        assert 0.0 < d["head_probs"][i].sum() <= 1.0 + 1e-6
        assert np.all(np.diff(d["head_probs"][i]) <= 0)
    assert d["rewards"].shape == (32,)


# --------------------------------------------------------------------------
# LM-head logits z = X W^T
# --------------------------------------------------------------------------
def test_lmhead_logits_one_hot_rows_select_weight_columns():
    # a one-hot hidden state e_j scores every id v by W[v, j]: catches a
    # transposed operand or a swapped contraction axis
    rng = np.random.default_rng(31)
    V, d = 7, 5
    W = rng.normal(0, 1, (V, d))
    X = np.eye(d)
    z = O.lmhead_logits(X, W)
    assert z.shape == (d, V)
    np.testing.assert_array_equal(z, W.T)


def test_lmhead_logits_gram_diagonal_and_scaling():
    rng = np.random.default_rng(32)
    W = rng.normal(0, 1, (6, 9))
    z = O.lmhead_logits(W, W)
    np.testing.assert_allclose(np.diag(z), np.sum(W * W, axis=1), rtol=1e-14)
    np.testing.assert_allclose(z, z.T, rtol=1e-14)
    X = rng.normal(0, 1, (3, 9))
    np.testing.assert_allclose(O.lmhead_logits(2.0 * X, W), 2.0 * O.lmhead_logits(X, W),
                               rtol=1e-14)
    with pytest.raises(ValueError):
        O.lmhead_logits(X, W[:, :8])


# --------------------------------------------------------------------------
# Rollout-side record: top-k candidates and the sampled token's log-prob
# --------------------------------------------------------------------------
def test_record_matches_torch_topk_on_distinct_logits():
    rng = np.random.default_rng(41)
    for T in (1.0, 0.6):
        z = rng.normal(0, 3, 5000)
        r = O.record_topk(z, T, 128, sampled=17)
        lp = torch.log_softmax(torch.tensor(z, dtype=torch.float64) / T, 0)
        top = torch.topk(lp, 128)
        np.testing.assert_array_equal(r["head_ids"], top.indices.numpy())
        np.testing.assert_allclose(r["head_probs"], top.values.exp().numpy(), rtol=1e-12)
        assert abs(r["sampled_logp"] - float(lp[17])) < 1e-12
        assert np.all(np.diff(r["head_probs"]) <= 0)


def test_record_ties_go_to_the_lower_id_and_probs_keep_normalisation():
    z = np.zeros(300)
    r = O.record_topk(z, 1.0, 10)
    np.testing.assert_array_equal(r["head_ids"], np.arange(10))
    np.testing.assert_allclose(r["head_probs"], np.full(10, 1 / 300), rtol=1e-14)
    # a tie group straddling the cut: ids 5, 9, 200 share the 2nd largest logit
    z = np.full(400, -1.0)
    z[[5, 9, 200]] = 2.0
    z[300] = 3.0
    r = O.record_topk(z, 1.0, 3)
    np.testing.assert_array_equal(r["head_ids"], [300, 5, 9])
    # k = V records everything: the probabilities sum to one
    z = np.random.default_rng(2).normal(0, 1, 64)
    r = O.record_topk(z, 0.8, 64)
    assert abs(r["head_probs"].sum() - 1.0) < 1e-12
    assert sorted(r["head_ids"].tolist()) == list(range(64))


def test_record_shift_invariance_and_temperature_scaling():
    rng = np.random.default_rng(43)
    z = rng.normal(0, 2, 1000)
    a = O.record_topk(z, 0.5, 50, sampled=3)
    b = O.record_topk(z + 7.25, 0.5, 50, sampled=3)
    c = O.record_topk(z / 0.5, 1.0, 50, sampled=3)
    for o in (b, c):
        np.testing.assert_array_equal(a["head_ids"], o["head_ids"])
        np.testing.assert_allclose(a["head_probs"], o["head_probs"], rtol=1e-12)
        assert abs(a["sampled_logp"] - o["sampled_logp"]) < 1e-12


def test_record_flags_and_masked_logits():
    z = np.zeros(10)
    z[4] = np.nan
    assert O.record_topk(z, 1.0, 3)["flags"] == O.DEV_NONFINITE
    assert O.record_topk(np.full(5, -np.inf), 1.0, 2)["flags"] == O.DEV_NONFINITE
    assert O.record_topk(np.zeros(5), 1.0, 2, sampled=5)["flags"] == O.DEV_BAD_SAMPLED
    z = np.array([0.0, -np.inf, 1.0, -np.inf])
    assert O.record_topk(z, 1.0, 2, sampled=1)["flags"] == O.DEV_NONFINITE
    r = O.record_topk(z, 1.0, 4, sampled=0)      # -inf entries fill the tail, p = 0
    np.testing.assert_array_equal(r["head_ids"], [2, 0, 1, 3])
    assert r["head_probs"][2] == 0.0 and r["head_probs"][3] == 0.0


def test_lmhead_backward_equals_autograd_of_printed_loss_through_the_head():
    # end to end: the printed token loss of every row, on logits X W^T, summed
    # over rows with the global token mean; torch autograd gives dX and dW
    rng = np.random.default_rng(51)
    n, V, d, T = 6, 12, 5, 0.8
    X = rng.normal(0, 1, (n, d))
    W = rng.normal(0, 0.7, (V, d))
    Xt = torch.tensor(X, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    z = Xt @ Wt.T / 1.0
    rows, total = [], 0.0
    cases = []
    for i in range(n):
        K = int(rng.integers(1, V))
        ids = rng.choice(V, K, replace=False)
        q = rng.dirichlet(np.ones(K)) * rng.uniform(0.3, 0.99)
        a = int(rng.integers(V))
        A = float(rng.normal())
        cases.append((ids, q, a, A))
        total = total + _printed_loss(z[i], T, torch.tensor(ids), torch.tensor(q), a, A, n)
    total.backward()
    zn = O.lmhead_logits(X, W)
    G = np.stack([O.sc_row(zn[i], T, ids, q, a, advantage=A, n_valid=n)["row"]
                  for i, (ids, q, a, A) in enumerate(cases)])
    dX, dW = O.lmhead_backward(X, W, G)
    np.testing.assert_allclose(dX, Xt.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-9, atol=1e-11)
    assert dX.shape == (n, d) and dW.shape == (V, d)
