"""Element-by-element comparison of the HIP path with the CPU oracle.

Tolerances (derived from the kernels' fp32 arithmetic; the oracle is exact
float64):

* log-probabilities (lse, log p(a), log p at H): abs 1e-5.  The kernel's
  exponent (z - m) log2(e) / T is rounded once in fp32, the sum of exps is an
  fp32 sum, and the log is taken in fp32.
* masses P_H, tau, Q_H, S and TV: abs 1e-6.
* rho: rel 1e-5 (tau carries the fp32 sum's relative error; the clamp
  max(tau, 1e-6) does not increase it).
* c_k = q_k - rho p_k: abs 1e-6 + 1e-5 |rho p_k| (rho's relative error scales
  the product, which reaches ~1e2 on clamp-active rows).
* loss: the propagated bound |A| (1e-5 + sum_k tol(c_k) |log p_k| + |c_k| 1e-5).
* KL: abs 1e-6 + rel 1e-5; K3: abs 1e-6 + 1e-5 |exp(d) - 1| (d has abs 1e-5).
* entropy ln s + (-D) / (T s): both parts are >= 0 and each carries the
  fp32 sums' relative error, so abs 1e-5 + rel 1e-5.
* importance ratio w = exp(d): rel 2e-5 (d has abs 1e-5, expf adds ulps);
  the weight takes w's tolerance, except that a masked-IS decision within
  that tolerance of a boundary may go either way (both outcomes checked
  valid).  The loss and the rows of a weighted token add the weight's
  relative error to their own.
* reverse KL sum_H p (log p - log q) - tau log rho: abs 1e-5 + 1e-6 |log rho|
  + 1e-5 sum_H p |log p - log q|; +inf (p > 0 where q = 0) exactly.
* full-vocabulary rows in fp32: abs 1e-6 |scale| + 4e-6 |value|.  Each entry
  is a single exp2 of an fp32 fused multiply-add of size |y| <= ~90, whose
  rounding gives a relative error <= (|y| 2^-24 + 4 2^-24) ln 2 < 4e-6.
* full-vocabulary rows in bf16: every entry within one bf16 step of the
  round-to-nearest-even of the float64 value, and at least 99.8% of them
  bit-equal (a relative error eps flips a rounding with probability at most
  2^9 eps <= 1.4e-3).
* argmax, a_slot and device flags: exact.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import sc_oracle as O

STAT_COLS = dict(lse=0, logp_a=1, tau=2, P_H=3, Q_H=4, rho=5, S=6, loss=7,
                 tv=8, kl=9, k3=10, entropy=11, w=12, weight=13, rev_kl=14)
REL_W = 2e-5


def bf16_bits_to_f64(bits):
    b = np.asarray(bits).astype(np.uint32) & 0xFFFF
    return (b << 16).view(np.float32).astype(np.float64)


def _ordered(x64):
    """Monotonic integer order of bf16 values given as float64."""
    f = x64.astype(np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def compare_bf16(gpu_bits, oracle_vals):
    """(max step distance, bit-equal fraction) of bf16 output vs RNE(oracle)."""
    ref = O.bf16_rne(oracle_vals)
    got = bf16_bits_to_f64(gpu_bits)
    both_nan = np.isnan(ref) & np.isnan(got)
    d = np.abs(_ordered(got) - _ordered(ref))
    d = np.where(both_nan, 0, d)
    eq = (got == ref) | both_nan
    return int(d.max()) if d.size else 0, float(eq.mean()) if eq.size else 1.0


def oracle_row(z, T, ids, q, a, rlp, A, n_valid, mode, **weighting):
    return O.sc_row(z, T, ids, q, a, rollout_logp=rlp, advantage=A,
                    n_valid=n_valid, row_mode=mode, **weighting)


def _gpu_weight(o, got_w, is_mode, is_lo, is_hi):
    """The weight the oracle assigns, with a masked-IS decision that falls
    within w's tolerance of a boundary taken from the GPU's own w."""
    if is_mode != O.IS_MIS:
        return o["weight"], False
    w = o["w"]
    near = min(abs(w - is_lo), abs(w - is_hi)) <= REL_W * abs(w) + 1e-12
    if not near:
        return o["weight"], False
    return O.is_weight(float(got_w), is_mode, is_lo, is_hi), True


def check_row(tag, g, o, A=1.0, T=1.0, n_valid=1, mode=O.MODE_DLOGITS,
              row_dtype=None, bf16_stats=None, stats_only=False, rlp=None,
              is_mode=O.IS_NONE, is_lo=0.5, is_hi=2.0, centering=True,
              rerun=None):
    """Assert one row's GPU outputs against the oracle dict ``o``.

    g: dict with numpy arrays: stats [16], idx [2], head_logp [K] and, unless
    stats_only, coef [K] and (when row_dtype) row [V] (fp32 values or bf16
    bits).  bf16_stats: list collecting (max_dist, equal_fraction).  The
    weighting arguments are the ones the oracle row was computed with;
    rerun(**overrides) recomputes the oracle row with other weighting
    arguments (needed only for a masked-IS decision at a boundary).
    """
    st = g["stats"]
    if o["flags"]:
        assert np.all(np.isnan(st[[0, 1, 2, 3]])), tag
        assert list(g["idx"]) == [-1, -1], tag
        return
    assert g["idx"][0] == o["argmax"], (tag, g["idx"][0], o["argmax"])
    assert g["idx"][1] == o["a_slot"], (tag, g["idx"][1], o["a_slot"])

    def close(name, got, want, tol):
        err = np.max(np.abs(np.asarray(got, np.float64) - want) - tol)
        assert err <= 0, (tag, name, np.max(np.abs(np.asarray(got, np.float64) - want)))

    close("lse", st[0], o["lse"], 1e-5)
    close("logp_a", st[1], o["logp_a"], 1e-5)
    close("tau", st[2], o["tau"], 1e-6)
    close("P_H", st[3], o["P_H"], 1e-6)
    close("head_logp", g["head_logp"], o["head_logp"], 1e-5)
    close("entropy", st[11], o["entropy"], 1e-5 + 1e-5 * abs(o["entropy"]))
    if stats_only:
        return
    close("Q_H", st[4], o["Q_H"], 1e-6)
    close("rho", st[5], o["rho"], 1e-5 * abs(o["rho"]))
    close("S", st[6], o["S"], 1e-6)
    p_h = np.exp(o["head_logp"])
    tol_c = 1e-6 + 1e-5 * np.abs(o["rho"] * p_h)
    close("coef", g["coef"], o["coef"], tol_c)
    if rlp is not None:
        close("w", st[12], o["w"], REL_W * abs(o["w"]))
    wt, boundary = _gpu_weight(o, st[12], is_mode, is_lo, is_hi)
    rel_wt = REL_W if (is_mode != O.IS_NONE and wt != 0) else 0.0
    close("weight", st[13], wt, rel_wt * abs(wt))
    if centering:
        bracket = o["logp_a"] - float(np.sum(o["coef"] * o["head_logp"]))
        tol_b = (1e-5 + np.sum(tol_c * np.abs(o["head_logp"]))
                 + np.sum(np.abs(o["coef"])) * 1e-5)
    else:
        bracket, tol_b = o["logp_a"], 1e-5
    loss = -A * wt * bracket
    tol_loss = abs(A) * (abs(wt) * tol_b + rel_wt * abs(wt * bracket))
    close("loss", st[7], loss, tol_loss)
    close("tv", st[8], o["tv"], 1e-6)
    close("kl", st[9], o["kl"], 1e-6 + 1e-5 * abs(o["kl"]))
    if math.isinf(o["rev_kl"]):
        assert st[14] == o["rev_kl"], (tag, "rev_kl", st[14])
    else:
        lq = np.log(np.where(o["coef"] + o["rho"] * p_h > 0,
                             o["coef"] + o["rho"] * p_h, 1.0))
        spread = float(np.sum(p_h * np.abs(o["head_logp"] - lq)))
        close("rev_kl", st[14], o["rev_kl"],
              1e-5 + 1e-6 * abs(math.log(o["rho"])) + 1e-5 * spread)
    if rlp is not None:
        d = o["logp_a"] - float(rlp)
        close("k3", st[10], o["k3"], 1e-6 + 1e-5 * abs(math.expm1(d)))
    if row_dtype is None:
        return
    ref_row = o["row"]
    if boundary and wt != o["weight"] and mode != O.MODE_CORRECTION:
        # The GPU took the other side of a masked-IS boundary: compare with
        # the oracle row at that weight (w itself, i.e. no cap, or zero).
        assert rerun is not None, (tag, "masked-IS boundary row needs rerun")
        ref_row = (rerun(is_mode=O.IS_TIS, is_hi=math.inf)["row"] if wt != 0
                   else o["row"] * 0.0)
    if mode == O.MODE_DLOGITS:
        scale = abs(A) / (T * n_valid)
    else:
        scale = 1.0
    if mode != O.MODE_CORRECTION:
        scale *= abs(wt)
    rel_row = 4e-6 + (rel_wt if mode != O.MODE_CORRECTION else 0.0)
    if row_dtype == "f32":
        tol = 1e-6 * scale + rel_row * np.abs(ref_row)
        close("row", g["row"], ref_row, tol)
    else:
        dist, eq = compare_bf16(g["row"], ref_row)
        assert dist <= 1, (tag, "bf16 row step distance", dist)
        if bf16_stats is not None:
            bf16_stats.append((dist, eq, ref_row.size))

