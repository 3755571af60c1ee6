"""Element-by-element comparison of the HIP path with the CPU oracle.

The bar is the one stated for this path (GPU result against the float64
oracle, per row):

* argmax, a_slot and device flags: exact.
* log-probabilities (lse, log p(a), log p at H): abs 1e-5.
* masses tau, P_H, Q_H, S and TV: abs 1e-6.
* rho: rel 1e-5.
* c_k = q_k - rho p_k: abs 1e-6, plus p_k times an error of rho of 2^-21
  relative (RHO_REL, below).
* K3: abs 1e-6.
* KL(mu_hat || p): abs 1e-6 + rel 1e-5.
* loss per row: abs 1e-4, plus |A wt| sum_k p_k |log p_k| times the same
  error of rho (the centering sum of c_k log p_k).
* full-vocabulary rows in fp32 (the score g, the correction mu_hat - p, or
  dLogits = -A wt / (T N_valid) g): abs 1e-6 per entry, scaled by the factor
  in front of g (|A wt| / (T N_valid) for dLogits, |wt| for the score).
* full-vocabulary rows in bf16: every entry within one bf16 step of the
  round-to-nearest-even of the float64 value, and at least 99.99% of the
  entries a test checks bit-equal.  An entry whose value is within
  |scale| 2^-45 of the float64 one counts as agreeing: the recorded entries
  are [k = a] - q_k - (1 - S) p_k (or q_k - p_k), and where q_k equals p_k to
  within 1e-15 that difference cancels to the size of the float64 rounding
  of S, a 128-term sum, in the oracle as in the kernel (~1e-16), so no
  implementation fixes its bits.  The floor is |scale| |lse| 2^-47 where that
  is larger: the two-call path hands lse over as an fp32 pair (48 bits), so
  each p_v it forms carries |lse| 2^-48 of relative error, and where the
  sampled entry 1 - p_a cancels to (nearly) zero, as in a one-id vocabulary or
  a row whose p_a is within 1e-13 of 1, that error is what is left.  And it
  adds |scale| p_v 2^-22 per entry where the row's p is at hand: p_v =
  2^(z c - E) / s with s the row's sum of V exponentials evaluated in fp32,
  whose relative error is a few 2^-24, so an entry carries that times p_v; it
  is far below one bf16 step of any entry that does not cancel, and decides
  only entries such as a recorded q_k within ~1e-7 of p_k.

Every output is an fp32 number, whose own spacing exceeds an absolute bound
once the value is large (2^-23 |x| > 1e-6 for |x| >= 16): an absolute
tolerance is therefore read as "abs tol, or one fp32 spacing of the exact
value where that is larger" (``f32_tol``); below |x| = 8 this is the
absolute tolerance itself.  For the log-probabilities (abs 1e-5) the spacing
takes over at |x| >= 128, e.g. log p of a recorded id far below the row
maximum at a low temperature.

rho = (1 - Q_H) / tau is ill-conditioned where tau is small under a large
leftover mass 1 - Q_H (the stated bar itself checks rho relative to 1e-5 only
while min(1 - Q_H, tau) >= 1e-4).  tau is a sum of exponentials evaluated in
fp32, each term within about two fp32 units of its value and the partial sums
in fp32, and the two-call path hands it over as an fp32 number: its relative
error is a few 2^-24, and rho carries it.  Where rho p_k is large, c_k and the
loss carry that error times rho p_k, beyond what abs 1e-6 and abs 1e-4 allow;
their bars add it at RHO_REL = 2^-21.  Where rho p_k <= 2 (every row whose
tail is not far smaller than 1 - Q_H) the added term is below 1e-6, and below
the clamp (tau < 1e-6) rho has no such error and nothing is added.

Extra signals, beyond the stated bar: entropy abs 1e-5 + rel 1e-6; the
importance ratio w and the weight rel 1e-6, or one fp32 spacing of the value
where that is larger (w = exp(log p(a) - log mu(a)) is formed in float64 from
log p(a), whose own error is far below 1e-6, and stored as fp32: a ratio below
the fp32 subnormal range stores as 0); reverse
KL abs 1e-6 + rel 1e-5.  A masked-IS decision within w's tolerance of a bound
may go either way (the test then checks the GPU's side against the oracle
row at that weight).
"""
from __future__ import annotations

import math

import numpy as np

from oracle import sc_oracle as O

STAT_COLS = dict(lse=0, logp_a=1, tau=2, P_H=3, Q_H=4, rho=5, S=6, loss=7,
                 tv=8, kl=9, k3=10, entropy=11, w=12, weight=13, rev_kl=14)
REL_W = 1e-6
RHO_REL = 2.0 ** -21
MIN_BF16_EQUAL = 0.9999

# Largest error seen per quantity, in units of its tolerance (printed by the
# tests that check many rows, for the record of how close the bar is).
WORST = {}


def f32_tol(want, atol):
    """abs tol, or one fp32 spacing of the value where that is larger."""
    w = np.abs(np.asarray(want, np.float64))
    sp = np.spacing(np.minimum(w, 3e38).astype(np.float32)).astype(np.float64)
    return np.maximum(atol, sp)


def f32_rel(want, rel):
    """rel |value|, or one fp32 spacing of the value where that is larger
    (a value below the fp32 subnormal range stores as 0 or the smallest
    subnormal, which no relative bound can ask more of)."""
    w = np.abs(np.asarray(want, np.float64))
    sp = np.spacing(np.minimum(w, 3e38).astype(np.float32)).astype(np.float64)
    return np.maximum(rel * w, sp)


def bf16_bits_to_f64(bits):
    b = np.asarray(bits).astype(np.uint32) & 0xFFFF
    return (b << 16).view(np.float32).astype(np.float64)


def _ordered(x64):
    """Monotonic integer order of bf16 values given as float64."""
    f = x64.astype(np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def compare_bf16(gpu_bits, oracle_vals, floor=0.0):
    """(max step distance, agreeing fraction) of bf16 output vs RNE(oracle).

    An entry agrees when its bits equal RNE(oracle), or when it lies within
    `floor` of the float64 value (see the module docstring)."""
    ref = O.bf16_rne(oracle_vals)
    got = bf16_bits_to_f64(gpu_bits)
    both_nan = np.isnan(ref) & np.isnan(got)
    near = np.abs(got - np.asarray(oracle_vals, np.float64)) <= floor
    d = np.abs(_ordered(got) - _ordered(ref))
    d = np.where(both_nan | near, 0, d)
    eq = (got == ref) | both_nan | near
    return int(d.max()) if d.size else 0, float(eq.mean()) if eq.size else 1.0


def bf16_bar(stats, tag):
    """Assert the bit-equal fraction over a test's bf16 entries.

    stats: list of (max_dist, equal_fraction, entries).  Returns the
    fraction.  The bar is MIN_BF16_EQUAL over all the entries the test
    checked."""
    total = sum(s[2] for s in stats)
    if not total:
        return 1.0
    eq = sum(s[1] * s[2] for s in stats) / total
    print(f"[case] {tag}: bf16 bit-equal fraction {eq:.7f} over {total} entries "
          f"({round((1 - eq) * total)} unequal)", flush=True)
    assert eq >= MIN_BF16_EQUAL, (tag, eq, total)
    return eq


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
              rerun=None, p_row=None):
    """Assert one row's GPU outputs against the oracle dict ``o``.

    g: dict with numpy arrays: stats [16], idx [2], head_logp [K] and, unless
    stats_only, coef [K] and (when row_dtype) row [V] (fp32 values or bf16
    bits).  bf16_stats: list collecting (max_dist, equal_fraction, entries).
    The weighting arguments are the ones the oracle row was computed with;
    rerun(**overrides) recomputes the oracle row with other weighting
    arguments (needed only for a masked-IS decision at a boundary).  p_row:
    the row's trainer probabilities (float64), for the bf16 floor of entries
    that cancel (see the module docstring).
    """
    st = g["stats"]
    if o["flags"]:
        assert np.all(np.isnan(st[[0, 1, 2, 3]])), tag
        assert list(g["idx"]) == [-1, -1], tag
        return
    assert g["idx"][0] == o["argmax"], (tag, g["idx"][0], o["argmax"])
    assert g["idx"][1] == o["a_slot"], (tag, g["idx"][1], o["a_slot"])

    def close(name, got, want, tol):
        err = np.abs(np.asarray(got, np.float64) - want)
        tol = np.broadcast_to(np.asarray(tol, np.float64), err.shape)
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = float(np.max(np.where(err == 0, 0.0, err / tol), initial=0.0))
        if ratio == ratio:
            WORST[name] = max(WORST.get(name, 0.0), ratio)
        assert np.all(err <= tol), (tag, name, float(np.max(err)), ratio)

    close("lse", st[0], o["lse"], f32_tol(o["lse"], 1e-5))
    close("logp_a", st[1], o["logp_a"], f32_tol(o["logp_a"], 1e-5))
    close("tau", st[2], o["tau"], 1e-6)
    close("P_H", st[3], o["P_H"], 1e-6)
    close("head_logp", g["head_logp"], o["head_logp"], f32_tol(o["head_logp"], 1e-5))
    close("entropy", st[11], o["entropy"], 1e-5 + 1e-6 * abs(o["entropy"]))
    if stats_only:
        return
    close("Q_H", st[4], o["Q_H"], 1e-6)
    close("rho", st[5], o["rho"], 1e-5 * abs(o["rho"]))
    close("S", st[6], o["S"], 1e-6)
    p_h = np.exp(np.asarray(o["head_logp"], np.float64))
    # rho's error comes from tau's; below the clamp (tau < 1e-6, taken with a
    # margin for tau's own error) rho = max(1 - Q_H, 1e-6) / 1e-6 has none
    rho_rel = RHO_REL if o["tau"] >= 0.5e-6 else 0.0
    close("coef", g["coef"], o["coef"],
          f32_tol(o["coef"], 1e-6) + rho_rel * np.abs(o["rho"] * p_h))
    if rlp is not None:
        close("w", st[12], o["w"], f32_rel(o["w"], REL_W))
    wt, boundary = _gpu_weight(o, st[12], is_mode, is_lo, is_hi)
    rel_wt = REL_W if (is_mode != O.IS_NONE and wt != 0) else 0.0
    close("weight", st[13], wt, f32_rel(wt, rel_wt) if rel_wt else 0.0)
    bracket = o["logp_a"] - (float(np.sum(o["coef"] * o["head_logp"])) if centering else 0.0)
    loss = -A * wt * bracket
    rho_loss = (abs(A * wt) * rho_rel * abs(o["rho"]) *
                float(np.sum(p_h * np.abs(o["head_logp"]))) if centering else 0.0)
    close("loss", st[7], loss, f32_tol(loss, 1e-4) + rho_loss)
    close("tv", st[8], o["tv"], 1e-6)
    close("kl", st[9], o["kl"], 1e-6 + 1e-5 * abs(o["kl"]))
    if math.isinf(o["rev_kl"]):
        assert st[14] == o["rev_kl"], (tag, "rev_kl", st[14])
    else:
        close("rev_kl", st[14], o["rev_kl"], 1e-6 + 1e-5 * abs(o["rev_kl"]))
    if rlp is not None:
        close("k3", st[10], o["k3"], f32_tol(o["k3"], 1e-6))
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
    if row_dtype == "f32":
        close("row", g["row"], ref_row, f32_tol(ref_row, 1e-6 * scale))
    else:
        floor = scale * max(2.0 ** -45, abs(float(o["lse"])) * 2.0 ** -47)
        if p_row is not None:
            floor = floor + scale * 2.0 ** -22 * p_row
        dist, eq = compare_bf16(g["row"], ref_row, floor=floor)
        assert dist <= 1, (tag, "bf16 row step distance", dist)
        if bf16_stats is not None:
            bf16_stats.append((dist, eq, ref_row.size))
