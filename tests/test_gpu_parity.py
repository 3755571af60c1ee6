"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Every test prints the case it is about to run (flushed) before touching the
GPU.  Small cases compare every row and every element; the full-size
workloads compare seeded samples of rows, each row element by element.
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import sc_oracle as O
import synthetic
from tests.parity import WORST, bf16_bar, check_row, compare_bf16

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from off_policy_logit_amd import sc

DEV = "cuda:0"
MODES = {"dlogits": O.MODE_DLOGITS, "score": O.MODE_SCORE,
         "correction": O.MODE_CORRECTION}


def say(*a):
    print("[case]", *a, flush=True)


def to_dev(d):
    out = {}
    for k, v in d.items():
        if isinstance(v, np.ndarray):
            out[k] = torch.from_numpy(np.ascontiguousarray(v)).to(DEV)
        elif isinstance(v, torch.Tensor):
            out[k] = v.to(DEV)
        else:
            out[k] = v
    return out


def host_rows(t, rows):
    x = t[rows]
    if x.dtype == torch.bfloat16:
        x = x.float()
    return x.cpu().numpy()


def run_correct(d, adv, n_valid, T, mode, out_dtype, logits=None, **weighting):
    logits = d["logits"] if logits is None else logits
    n, V = logits.shape
    row_out = None
    if out_dtype is not None:
        row_out = torch.empty(n, V, device=DEV,
                              dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = sc.correct(logits, d["head_ids"], d["head_probs"], d["sampled"],
                     d["resp_idx"], adv, temperature=T, n_valid=n_valid,
                     rollout_logp=d["rollout_logp"], row_out=row_out,
                     row_mode=mode, dev_status=status, **weighting)
    out["row"] = row_out
    out["status"] = status
    return out


def gather(out, rows, out_dtype):
    g = dict(stats=host_rows(out["row_stats"], rows), idx=host_rows(out["row_idx"], rows),
             head_logp=host_rows(out["head_logp"], rows), coef=host_rows(out["coef"], rows))
    if out_dtype == "bf16":
        g["row"] = out["row"][rows].view(torch.int16).cpu().numpy()
    elif out_dtype == "f32":
        g["row"] = host_rows(out["row"], rows)
    return g


# Host threads for the oracle (numpy releases the interpreter lock in its
# large array operations); bounded by the CPU share of one GPU machine.
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


def check_rows(tag, d, out, rows, adv_h, n_valid, T, mode, out_dtype,
               logits_h=None, bf16_stats=None, **weighting):
    """Compare the listed rows of a GPU result with the oracle, one row per
    task on ORACLE_THREADS host threads.

    weighting: is_mode / is_lo / is_hi / centering, passed to both sides.
    bf16_stats: a list to collect the rows' bf16 statistics in (the caller
    then applies the bar over all of them); when None the bar is applied to
    these rows here.  Returns the oracle dicts of the valid rows by row."""
    rows = np.asarray(rows)
    T = float(np.float32(T))   # the temperature the library receives (fp32)
    z = logits_h if logits_h is not None else host_rows(d["logits"], rows)
    ids = host_rows(d["head_ids"], rows)
    q = host_rows(d["head_probs"], rows)
    a = host_rows(d["sampled"], rows)
    rlp = host_rows(d["rollout_logp"], rows)
    resp = host_rows(d["resp_idx"], rows)
    g = gather(out, rows, out_dtype)
    local = bf16_stats if bf16_stats is not None else []

    def one(j):
        r = rows[j]
        gj = {key: val[j] for key, val in g.items()}
        if resp[j] < 0:
            assert np.all(gj["stats"][:15] == 0) and list(gj["idx"]) == [-1, -1]
            if out_dtype is not None:
                assert np.all(gj["row"] == 0)
            return None
        A = float(adv_h[resp[j]])

        def rerun(j=j, A=A, **over):
            return O.sc_row(z[j], T, ids[j], q[j], a[j], rollout_logp=rlp[j],
                            advantage=A, n_valid=n_valid, row_mode=mode,
                            **dict(weighting, **over))
        o = rerun()
        st = []
        p_row = (np.exp(z[j].astype(np.float64) / T - o["lse"])
                 if out_dtype == "bf16" else None)
        check_row(f"{tag} row {r}", gj, o, A=A, T=T, n_valid=n_valid, mode=mode,
                  row_dtype=out_dtype, bf16_stats=st, rlp=rlp[j], rerun=rerun,
                  p_row=p_row, **weighting)
        o.pop("row")
        return int(r), o, st

    with ThreadPoolExecutor(ORACLE_THREADS) as ex:
        results = list(ex.map(one, range(len(rows))))
    found = {}
    for res in results:
        if res is None:
            continue
        r, o, st = res
        local.extend(st)
        found[r] = o
    if bf16_stats is None and local:
        bf16_bar(local, tag)
    return found


# ---------------------------------------------------------------------------
# Tiny workload: every row, every output, every row mode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T", [1.0, 0.7])
@pytest.mark.parametrize("mode,out_dtype", [("dlogits", "bf16"), ("score", "f32"),
                                            ("correction", "f32"), ("dlogits", "f32"),
                                            ("score", None)])
def test_tiny_all_rows_correct(T, mode, out_dtype):
    say(f"tiny 256x4096 fp32 T={T} sc_correct mode={mode} out={out_dtype}")
    h = synthetic.tiny(seed=0, temperature=T)
    d = to_dev(h)
    adv = sc.group_norm(d["rewards"], h["group_size"])
    n_valid = sc.count_valid(d["resp_idx"])
    out = run_correct(d, adv, n_valid, T, MODES[mode], out_dtype)
    torch.cuda.synchronize()
    assert int(out["status"].item()) == 0
    nv = int(n_valid.item())
    assert nv == 256
    adv_h = adv.cpu().numpy()
    np.testing.assert_allclose(adv_h, O.group_norm(h["rewards"], 4), atol=1e-6)
    check_rows(f"tiny T={T} {mode}/{out_dtype}", d, out, np.arange(256), adv_h, nv,
               T, MODES[mode], out_dtype, logits_h=h["logits"])


@pytest.mark.parametrize("out_dtype", ["bf16", "f32", None])
def test_tiny_two_call_path(out_dtype):
    say(f"tiny sc_logprobs + sc_center out={out_dtype}")
    h = synthetic.tiny(seed=4)
    d = to_dev(h)
    adv = sc.group_norm(d["rewards"], 4)
    n_valid = sc.count_valid(d["resp_idx"])
    st = sc.logprobs(d["logits"], d["head_ids"], d["sampled"], d["resp_idx"])
    torch.cuda.synchronize()
    # stats-only check of sc_logprobs
    rows = np.arange(256)
    z = h["logits"]
    for r in rows[::17]:
        o = O.sc_row(z[r], 1.0, h["head_ids"][r], h["head_probs"][r], h["sampled"][r])
        g = dict(stats=st["row_stats"][r].cpu().numpy(), idx=st["row_idx"][r].cpu().numpy(),
                 head_logp=st["head_logp"][r].cpu().numpy())
        check_row(f"logprobs row {r}", g, o, stats_only=True)
    row_out = None
    if out_dtype:
        row_out = torch.empty(256, 4096, device=DEV,
                              dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    sc.center(st, d["head_ids"], d["head_probs"], d["sampled"], d["resp_idx"], adv,
              n_valid=n_valid, rollout_logp=d["rollout_logp"], logits=d["logits"],
              row_out=row_out, dev_status=status)
    st["row"] = row_out
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    # the two-call path rounds lse to fp32 between the calls: a second
    # rounding of relative size |lse| 2^-24 enters every p_v
    check_rows(f"two-call {out_dtype}", d, st, rows, adv.cpu().numpy(), 256, 1.0,
               O.MODE_DLOGITS, out_dtype, logits_h=z)


# ---------------------------------------------------------------------------
# Ragged vocabulary, strided / misaligned rows (scalar path), K extremes
# ---------------------------------------------------------------------------
# ---------------------------------------------------------------------------
# Importance weighting (truncated / masked) and the uncentered ablation
# ---------------------------------------------------------------------------
IS_LO, IS_HI = 0.8, 1.25


def tiny_spread(seed):
    """Tiny workload whose rollout log-probabilities are shifted by N(0, 0.5)
    (capped at 0), so that importance ratios fall on both sides of
    [IS_LO, IS_HI]."""
    h = synthetic.tiny(seed=seed, temperature=0.8)
    rng = np.random.default_rng(seed + 100)
    shift = rng.normal(0.0, 0.5, h["rollout_logp"].shape)
    h["rollout_logp"] = np.minimum(h["rollout_logp"] + shift, 0.0).astype(np.float32)
    return h


@pytest.mark.parametrize("is_mode,centering", [(O.IS_TIS, True), (O.IS_MIS, True),
                                               (O.IS_MIS, False), (O.IS_NONE, False)])
@pytest.mark.parametrize("mode,out_dtype", [("dlogits", "f32"), ("score", "bf16")])
def test_tiny_importance_weighting(is_mode, centering, mode, out_dtype):
    say(f"tiny weighting is_mode={is_mode} centering={centering} {mode}/{out_dtype}")
    h = tiny_spread(3)
    d = to_dev(h)
    adv = sc.group_norm(d["rewards"], h["group_size"])
    n_valid = sc.count_valid(d["resp_idx"])
    wkw = dict(is_mode=is_mode, is_lo=IS_LO, is_hi=IS_HI, centering=centering)
    out = run_correct(d, adv, n_valid, 0.8, MODES[mode], out_dtype, **wkw)
    torch.cuda.synchronize()
    assert int(out["status"].item()) == 0
    check_rows(f"tiny weighting {is_mode}/{centering} {mode}/{out_dtype}", d, out,
               np.arange(256), adv.cpu().numpy(), 256, 0.8, MODES[mode], out_dtype,
               logits_h=h["logits"], **wkw)
    w = out["row_stats"][:, sc.STAT["w"]].cpu().numpy()
    assert (w < IS_LO).sum() >= 20 and (w > IS_HI).sum() >= 20
    assert ((w >= IS_LO) & (w <= IS_HI)).sum() >= 20


def test_tiny_two_call_weighting():
    say("tiny sc_logprobs + sc_center, masked IS, f32 dlogits")
    h = tiny_spread(4)
    d = to_dev(h)
    adv = sc.group_norm(d["rewards"], h["group_size"])
    n_valid = sc.count_valid(d["resp_idx"])
    wkw = dict(is_mode=O.IS_MIS, is_lo=IS_LO, is_hi=IS_HI, centering=True)
    st = sc.logprobs(d["logits"], d["head_ids"], d["sampled"], d["resp_idx"],
                     temperature=0.8)
    row_out = torch.empty(256, 4096, device=DEV)
    sc.center(st, d["head_ids"], d["head_probs"], d["sampled"], d["resp_idx"], adv,
              temperature=0.8, n_valid=n_valid, rollout_logp=d["rollout_logp"],
              logits=d["logits"], row_out=row_out, row_mode=O.MODE_DLOGITS, **wkw)
    st["row"] = row_out
    torch.cuda.synchronize()
    check_rows("tiny two-call MIS", d, st, np.arange(256), adv.cpu().numpy(), 256, 0.8,
               O.MODE_DLOGITS, "f32", logits_h=h["logits"], **wkw)


def crafted(n, V, K, seed, dtype, stride=None, scale=2.0):
    rng = np.random.default_rng(seed)
    z = rng.normal(0, scale, (n, V)).astype(np.float32)
    if dtype == "bf16":
        z = torch.from_numpy(z).to(torch.bfloat16).float().numpy()
    ids = np.stack([rng.choice(V, K, replace=False) for _ in range(n)]).astype(np.int32)
    q = (rng.dirichlet(np.ones(K), n) * rng.uniform(0.2, 0.999, (n, 1))).astype(np.float32)
    a = rng.integers(0, V, n).astype(np.int32)
    half = n // 2
    a[:half] = ids[np.arange(half), rng.integers(0, K, half)]   # some a inside H
    rlp = np.log(rng.uniform(0.01, 1.0, n)).astype(np.float32)
    resp = (np.arange(n) // 4).astype(np.int32)
    stride = stride or V
    buf = np.zeros((n, stride), np.float32)
    buf[:, :V] = z
    t = torch.from_numpy(buf).to(DEV)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    logits = t[:, :V]
    d = dict(logits=logits, head_ids=torch.from_numpy(ids).to(DEV),
             head_probs=torch.from_numpy(q).to(DEV), sampled=torch.from_numpy(a).to(DEV),
             rollout_logp=torch.from_numpy(rlp).to(DEV), resp_idx=torch.from_numpy(resp).to(DEV))
    return d, z


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V,K,stride", [(4099, 128, None), (4099, 128, 4100), (2000, 1, None),
                                        (200, 200, None), (1031, 129, 1040), (4099, 64, 4101), (63, 7, None),
                                        (8 * 1024 + 3, 1024, None)])
def test_ragged_strided_and_k_extremes(dtype, V, K, stride):
    say(f"crafted n=32 V={V} K={K} stride={stride} dtype={dtype}")
    d, z = crafted(32, V, K, seed=V + K, dtype=dtype, stride=stride)
    adv = torch.linspace(-1.5, 1.5, 8, device=DEV)
    n_valid = sc.count_valid(d["resp_idx"])
    for out_dtype in ("bf16", "f32"):
        out = run_correct(d, adv, n_valid, 1.0, O.MODE_SCORE, out_dtype)
        torch.cuda.synchronize()
        assert int(out["status"].item()) == 0
        check_rows(f"crafted V={V} K={K} {dtype}->{out_dtype}", d, out, np.arange(32),
                   adv.cpu().numpy(), 32, 1.0, O.MODE_SCORE, out_dtype, logits_h=z)


# ---------------------------------------------------------------------------
# Padding rows and data errors
# ---------------------------------------------------------------------------
def test_padding_rows_and_data_errors():
    say("crafted data-error rows V=1000 K=16 bf16")
    d, z = crafted(12, 1000, 16, seed=3, dtype="bf16")
    ids = d["head_ids"].cpu().numpy()
    a = d["sampled"].cpu().numpy()
    resp = d["resp_idx"].cpu().numpy()
    resp[1] = -1                        # padding
    ids[2, 3] = 1000                    # id out of range
    ids[3, 5] = ids[3, 6]               # duplicate id
    a[4] = -2                           # sampled out of range
    zl = z.copy()
    zl[5, 10] = np.nan                  # NaN logit
    zl[6, ids[6, 0]] = -np.inf          # -inf at a recorded id
    zl[7, 999] = -np.inf                # -inf elsewhere: legal
    if a[7] == 999 or 999 in ids[7]:
        zl[7, 998] = -np.inf
        zl[7, 999] = z[7, 999]
    resp[8] = 3                         # response index beyond advantages
    logits = torch.from_numpy(zl).to(DEV).to(torch.bfloat16)
    d.update(logits=logits, head_ids=torch.from_numpy(ids).to(DEV),
             sampled=torch.from_numpy(a).to(DEV), resp_idx=torch.from_numpy(resp).to(DEV))
    adv = torch.tensor([0.5, -1.0, 2.0], device=DEV)   # resp 3 is out of range
    n_valid = sc.count_valid(d["resp_idx"])
    out = run_correct(d, adv, n_valid, 1.0, O.MODE_DLOGITS, "bf16")
    torch.cuda.synchronize()
    st = out["row_stats"].cpu().numpy()
    idx = out["row_idx"].cpu().numpy()
    row = out["row"].float().cpu().numpy()
    flags = int(out["status"].item())
    assert flags == (O.DEV_BAD_ID | O.DEV_DUP_ID | O.DEV_BAD_SAMPLED | O.DEV_NONFINITE
                     | O.DEV_BAD_RESP)
    assert np.all(st[1, :11] == 0) and np.all(row[1] == 0) and list(idx[1]) == [-1, -1]
    for r in (2, 3, 4, 5, 6, 8):
        assert np.all(np.isnan(st[r, [0, 1, 7]])), r
        assert list(idx[r]) == [-1, -1], r
        assert np.all(np.isnan(row[r])), r
    assert int(n_valid.item()) == 11
    # row 7 is valid: compare with the oracle
    o = O.sc_row(zl[7].astype(np.float64), 1.0, ids[7], d["head_probs"][7].cpu().numpy(),
                 a[7], rollout_logp=float(d["rollout_logp"][7]), advantage=-1.0,
                 n_valid=11)
    assert o["flags"] == 0
    g = dict(stats=st[7], idx=idx[7], head_logp=out["head_logp"][7].cpu().numpy(),
             coef=out["coef"][7].cpu().numpy(),
             row=out["row"][7].view(torch.int16).cpu().numpy())
    check_row("row 7 with -inf logit", g, o, A=-1.0, n_valid=11, row_dtype="bf16",
              rlp=float(d["rollout_logp"][7]))


# ---------------------------------------------------------------------------
# Group normalisation, counts, step sums
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("G", [1, 4, 8, 33])
def test_group_norm_matches_oracle(mode, G):
    say(f"group_norm G={G} mode={mode}")
    rng = np.random.default_rng(G * 10 + mode)
    r = np.concatenate([
        (rng.random(G * 16) < 0.5).astype(np.float32),
        rng.normal(0, 1, G * 16).astype(np.float32),
        np.full(G, 0.25, np.float32),
        np.tile(np.array([1.0, 1.001], np.float32), G)[:G],
        (rng.normal(0, 1, G) * 1e30).astype(np.float32),
    ])
    got = sc.group_norm(torch.from_numpy(r).to(DEV), G, mode=mode).cpu().numpy()
    want = O.group_norm(r, G, mode=mode)
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-6)
    assert np.all(got[G * 32:G * 33] == 0)
    if G > 1 and mode != 2:
        pair = got[G * 33:G * 34]
        assert len(set(pair.tolist())) == 2


def test_count_valid_and_batch_sums():
    say("count_valid / batch_sums on 3 chunks")
    rng = np.random.default_rng(11)
    n = 5000
    chunks = []
    for c in range(3):
        resp = rng.integers(-1, 7, n).astype(np.int32)
        st = rng.normal(0, 1, (n, sc.NSTATS)).astype(np.float32)
        st[:, sc.STAT["w"]] = np.exp(st[:, sc.STAT["w"]])
        chunks.append((resp, st))
    total = sum(int((r >= 0).sum()) for r, _ in chunks)
    nv = torch.zeros(1, dtype=torch.int64, device=DEV)
    for i, (resp, _) in enumerate(chunks):
        sc.count_valid(torch.from_numpy(resp).to(DEV), out=nv, accumulate=i > 0)
    assert int(nv.item()) == total
    batch = torch.zeros(sc.NBATCH, dtype=torch.float64, device=DEV)
    for i, (resp, st) in enumerate(chunks):
        sc.batch_sums(torch.from_numpy(st).to(DEV), torch.from_numpy(resp).to(DEV), nv,
                      out=batch, accumulate=i > 0)
    b = batch.cpu().numpy()
    rows = [dict(loss=s[7], k3=s[10], tv=s[8], kl=s[9], Q_H=s[4], P_H=s[3],
                 entropy=s[11], rev_kl=s[14], w=s[12])
            for resp, st in chunks for s, r in zip(st, resp) if r >= 0]
    sums, means = O.batch_sums(rows, total)
    B = sc.BATCH.index
    for key in O.BATCH_KEYS:
        got_s, got_m = b[B("sum_" + key)], b[B("mean_" + key)]
        assert abs(got_s - sums[key]) <= 1e-9 * max(1, abs(sums[key])), key
        assert abs(got_m - means[key]) <= 1e-12 * max(1, abs(means[key])), key
    assert b[B("rows")] == total and b[B("flagged")] == 0
    assert b[B("max_w")] == np.float32(means["max_w"])


def test_empty_chunks_in_the_step_reductions():
    """A chunk with no rows adds nothing to the count or the step sums, and a
    fresh (non-accumulating) pass over no rows gives what the oracle's step
    reduction gives over an empty set: zero count and sums, no maximum
    weight."""
    say("count_valid / batch_sums with empty chunks")
    rng = np.random.default_rng(12)
    n = 3000
    resp = torch.from_numpy(rng.integers(-1, 5, n).astype(np.int32)).to(DEV)
    st = torch.from_numpy(rng.normal(0, 1, (n, sc.NSTATS)).astype(np.float32)).to(DEV)
    st[:, sc.STAT["w"]] = st[:, sc.STAT["w"]].exp()
    no_resp = torch.empty(0, dtype=torch.int32, device=DEV)
    no_st = torch.empty(0, sc.NSTATS, device=DEV)

    nv = torch.full((1,), 77, dtype=torch.int64, device=DEV)
    sc.count_valid(no_resp, out=nv)
    assert int(nv.item()) == 0
    sc.count_valid(resp, out=nv, accumulate=True)
    expect = int((resp >= 0).sum().item())
    sc.count_valid(no_resp, out=nv, accumulate=True)
    assert int(nv.item()) == expect

    one = sc.batch_sums(st, resp, nv)
    both = sc.batch_sums(st, resp, nv)
    sc.batch_sums(no_st, no_resp, nv, out=both, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(one, both)

    fresh = torch.full((sc.NBATCH,), 5.0, dtype=torch.float64, device=DEV)
    sc.batch_sums(no_st, no_resp, nv, out=fresh)
    f = fresh.cpu().numpy()
    sums, means = O.batch_sums([], expect)
    B = sc.BATCH.index
    assert f[B("rows")] == 0 and f[B("flagged")] == 0
    assert f[B("max_w")] == means["max_w"]
    for key in O.BATCH_KEYS:
        assert f[B("sum_" + key)] == sums[key] and f[B("mean_" + key)] == means[key], key


# ---------------------------------------------------------------------------
# Full-size workloads (V = 248,320), sampled rows
# ---------------------------------------------------------------------------
def sample_rows(n, count, seed, extra=()):
    """Rows 0 and n - 1, the `extra` rows, and seeded distinct others, sorted:
    exactly `count` rows (or n when count >= n)."""
    rng = np.random.default_rng(seed)
    fixed = sorted({0, n - 1} | set(int(e) for e in extra))[:count]
    rest = np.setdiff1d(np.arange(n), fixed)
    pick = rng.choice(rest, max(0, min(count, n) - len(fixed)), replace=False)
    return np.array(sorted(set(fixed) | set(pick.tolist())))


@pytest.fixture(scope="module")
def quick():
    say("generate quick-check workload 8192 x 248320 bf16")
    d = synthetic.quick_check(DEV)
    torch.cuda.synchronize()
    return d


def check_in_blocks(tag, d, out, rows, adv_h, n_valid, T, mode, out_dtype, stats,
                    block=512, **weighting):
    """check_rows over a long row list in blocks (bounded host memory)."""
    found = {}
    for b0 in range(0, len(rows), block):
        found.update(check_rows(tag, d, out, rows[b0:b0 + block], adv_h, n_valid, T, mode,
                                out_dtype, bf16_stats=stats, **weighting))
    return found


def test_quick_check_all_rows(quick):
    """The bench configuration (sc_correct, bf16 dLogits) on all 8,192
    quick-check rows, every output element against the oracle."""
    d = quick
    say("quick-check sc_correct bf16 dlogits (bench configuration), all 8192 rows")
    adv = sc.group_norm(d["rewards"], d["group_size"])
    n_valid = sc.count_valid(d["resp_idx"])
    out = run_correct(d, adv, n_valid, 1.0, O.MODE_DLOGITS, "bf16")
    torch.cuda.synchronize()
    assert int(out["status"].item()) == 0
    stats = []
    WORST.clear()
    check_in_blocks("quick-check dlogits bf16", d, out, np.arange(8192), adv.cpu().numpy(),
                    8192, 1.0, O.MODE_DLOGITS, "bf16", stats)
    bf16_bar(stats, "quick-check all rows")
    say("  worst error / tolerance: " + ", ".join(f"{k} {v:.3f}" for k, v in sorted(WORST.items())))
    # determinism: a second run is bitwise identical
    out2 = run_correct(d, adv, n_valid, 1.0, O.MODE_DLOGITS, "bf16")
    torch.cuda.synchronize()
    for key in ("row_stats", "row_idx", "head_logp", "coef"):
        assert torch.equal(out[key].view(torch.int32), out2[key].view(torch.int32)), key
    assert torch.equal(out["row"].view(torch.int16), out2["row"].view(torch.int16))
    # argmax and a_slot of every row against torch on the same logits
    am = torch.argmax(d["logits"].float(), dim=1).to(torch.int32)
    assert torch.equal(out["row_idx"][:, 0], am)
    hit = (d["head_ids"] == d["sampled"][:, None])
    slot = torch.where(hit.any(1), hit.int().argmax(1), torch.full_like(am, -1)).to(torch.int32)
    assert torch.equal(out["row_idx"][:, 1], slot)


def test_quick_check_two_call_and_f32_rows(quick):
    d = quick
    say("quick-check sc_logprobs + sc_center f32 score rows")
    adv = sc.group_norm(d["rewards"], d["group_size"])
    n_valid = sc.count_valid(d["resp_idx"])
    st = sc.logprobs(d["logits"], d["head_ids"], d["sampled"], d["resp_idx"])
    rows = sample_rows(8192, 64, seed=22)
    sub = torch.as_tensor(rows, device=DEV)
    dd = {k: (v[sub] if isinstance(v, torch.Tensor) and v.shape[0] == 8192 else v)
          for k, v in d.items()}
    stt = {k: v[sub].contiguous() for k, v in st.items()}
    row_out = torch.empty(len(rows), synthetic.VOCAB, device=DEV)
    sc.center(stt, dd["head_ids"].contiguous(), dd["head_probs"].contiguous(),
              dd["sampled"].contiguous(), dd["resp_idx"].contiguous(), adv,
              n_valid=n_valid, rollout_logp=dd["rollout_logp"].contiguous(),
              logits=dd["logits"].contiguous(), row_out=row_out, row_mode=O.MODE_SCORE)
    stt["row"] = row_out
    torch.cuda.synchronize()
    check_rows("quick-check two-call score f32", dd, stt, np.arange(len(rows)),
               adv.cpu().numpy(), 8192, 1.0, O.MODE_SCORE, "f32")


def test_quick_check_masked_is_and_step_sums(quick):
    d = quick
    say("quick-check sc_correct bf16 dlogits, masked IS, then batch_sums")
    adv = sc.group_norm(d["rewards"], d["group_size"])
    n_valid = sc.count_valid(d["resp_idx"])
    wkw = dict(is_mode=O.IS_MIS, is_lo=0.99, is_hi=1.01, centering=True)
    out = run_correct(d, adv, n_valid, 1.0, O.MODE_DLOGITS, "bf16", **wkw)
    batch = sc.batch_sums(out["row_stats"], d["resp_idx"], n_valid)
    torch.cuda.synchronize()
    assert int(out["status"].item()) == 0
    rows = sample_rows(8192, 256, seed=24)
    check_rows("quick-check MIS dlogits bf16", d, out, rows, adv.cpu().numpy(), 8192,
               1.0, O.MODE_DLOGITS, "bf16", **wkw)
    st = out["row_stats"].double().cpu().numpy()
    b = batch.cpu().numpy()
    B = sc.BATCH.index
    assert b[B("max_w")] == st[:, sc.STAT["w"]].max()
    assert b[B("rows")] == 8192 and b[B("flagged")] == 0
    for key in ("entropy", "rev_kl", "loss"):
        ref = math.fsum(st[:, sc.STAT[key]])
        assert abs(b[B("sum_" + key)] - ref) <= 1e-9 * max(1.0, abs(ref)), key


def test_full_step_all_chunks_sampled():
    """The full-step workload (32 prompts x 4 responses x 4,096 tokens,
    lengths uniform in [256, 4,096], padding masked) in its 32 chunks of
    16,384 rows: 128 seeded rows of every chunk (4,096 in all, padding rows
    included) against the oracle, with N_valid counted over the whole step
    by accumulating sc_count_valid chunk by chunk."""
    lengths = synthetic.full_step_lengths()
    n_valid_total = int(np.sum(np.minimum(lengths, 4096)))
    rewards = torch.from_numpy(
        (np.random.default_rng(2).random(128) < 0.5).astype(np.float32)).to(DEV)
    adv = sc.group_norm(rewards, 4)
    adv_h = adv.cpu().numpy()
    nv = torch.zeros(1, dtype=torch.int64, device=DEV)
    for c in range(32):
        rows = torch.arange(c * 16384, (c + 1) * 16384)
        lens = torch.as_tensor(lengths)[rows // 4096]
        resp = torch.where(rows % 4096 < lens, rows // 4096, -1).to(torch.int32).to(DEV)
        sc.count_valid(resp, out=nv, accumulate=c > 0)
    assert int(nv.item()) == n_valid_total
    stats, checked, padded = [], 0, 0
    for c in range(32):
        say(f"full-step chunk {c} of 32 (16384 rows, padded responses)")
        d = synthetic.full_step_chunk(DEV, c, lengths)
        out = run_correct(d, adv, nv, 1.0, O.MODE_DLOGITS, "bf16")
        torch.cuda.synchronize()
        assert int(out["status"].item()) == 0
        resp_h = d["resp_idx"].cpu().numpy()
        pad = np.nonzero(resp_h < 0)[0]
        rows = sample_rows(16384, 128, seed=230 + c, extra=pad[:1].tolist())
        found = check_rows(f"full-step chunk {c}", d, out, rows, adv_h, n_valid_total, 1.0,
                           O.MODE_DLOGITS, "bf16", bf16_stats=stats)
        checked += len(rows)
        padded += len(rows) - len(found)
        del d, out
    say(f"full-step: {checked} rows checked over 32 chunks, {padded} of them padding")
    assert checked == 4096 and padded >= 32
    bf16_bar(stats, "full-step 32 chunks")


@pytest.mark.parametrize("sigma", [0.01, 0.1, 0.5])
def test_stress_all_chunks_sampled(sigma):
    """Distribution stress (131,072 rows at rollout noise sigma: peaked, flat
    and mixed rows, 5% of samples outside the head) in its 8 chunks of
    16,384 rows: 512 seeded rows of every chunk (4,096 in all) against the
    oracle, in the centered-score mode.  The sample must hold clamp-active
    rows (tau < 1e-6 or 1 - Q_H < 1e-6) and sampled tokens outside H."""
    stats, clamp, ooh, total = [], 0, 0, 0
    WORST.clear()
    adv = torch.tensor([1.0], device=DEV)
    n_valid = torch.tensor([131072], dtype=torch.int64, device=DEV)
    for c in range(8):
        say(f"distribution stress sigma={sigma} chunk {c} of 8 (16384 rows)")
        d = synthetic.stress_chunk(DEV, c, sigma)
        out = run_correct(d, adv, n_valid, 1.0, O.MODE_SCORE, "bf16")
        torch.cuda.synchronize()
        assert int(out["status"].item()) == 0
        rows = sample_rows(16384, 512, seed=int(sigma * 1000) + c)
        found = check_rows(f"stress sigma={sigma} chunk {c}", d, out, rows, np.array([1.0]),
                           131072, 1.0, O.MODE_SCORE, "bf16", bf16_stats=stats)
        for o in found.values():
            clamp += (o["tau"] < 1e-6) or (1.0 - o["Q_H"] < 1e-6)
            ooh += o["a_slot"] < 0
        total += len(found)
        del d, out
    say(f"stress sigma={sigma}: {total} rows checked, {clamp} clamp-active, "
        f"{ooh} sampled outside H")
    say("  worst error / tolerance: " + ", ".join(f"{k} {v:.3f}" for k, v in sorted(WORST.items())))
    assert total == 4096 and clamp >= 100 and ooh >= 100
    bf16_bar(stats, f"stress sigma={sigma} 8 chunks")


def clamp_corner_rows(kind, n, V, K, seed, dtype):
    """Rows at the two corners of rho's clamps (Score Centering section: rho
    with 1e-6 in numerator and denominator).

    "tiny_tau": the trainer puts all but ~1e-7 of its mass on the recorded
    ids (tau < 1e-6, the denominator clamp) while the recorded mass Q_H is at
    most 0.9, so S = Q_H + rho tau < 0.95 and the score departs from
    e_a - mu_hat by (1 - S) p.  "q_ge_1": recorded probabilities that sum to
    1 or just above it (the numerator clamp)."""
    rng = np.random.default_rng(seed)
    z = rng.normal(0, 1, (n, V)).astype(np.float32)
    ids = np.stack([rng.choice(V, K, replace=False) for _ in range(n)]).astype(np.int32)
    if kind == "tiny_tau":
        for r in range(n):
            z[r, ids[r]] += 20.0 + rng.normal(0, 1, K).astype(np.float32)
        q = rng.dirichlet(np.ones(K), n) * rng.uniform(0.5, 0.9, (n, 1))
    else:
        q = rng.dirichlet(np.ones(K), n)
        q[n // 2:] *= 1.0 + 2.0 ** -21
    q = q.astype(np.float32)
    if dtype == "bf16":
        z = torch.from_numpy(z).to(torch.bfloat16).float().numpy()
    a = rng.integers(0, V, n).astype(np.int32)
    a[::2] = ids[np.arange(0, n, 2), rng.integers(0, K, (n + 1) // 2)]
    rlp = np.log(rng.uniform(0.05, 1.0, n)).astype(np.float32)
    resp = (np.arange(n) // 4).astype(np.int32)
    t = torch.from_numpy(z).to(DEV)
    d = dict(logits=t.to(torch.bfloat16) if dtype == "bf16" else t,
             head_ids=torch.from_numpy(ids).to(DEV), head_probs=torch.from_numpy(q).to(DEV),
             sampled=torch.from_numpy(a).to(DEV), rollout_logp=torch.from_numpy(rlp).to(DEV),
             resp_idx=torch.from_numpy(resp).to(DEV))
    return d, z


@pytest.mark.parametrize("kind", ["tiny_tau", "q_ge_1"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_clamp_corners(kind, dtype):
    """Both clamp corners in all three row modes and both output dtypes."""
    n, V, K = 32, 4099, 64
    d, z = clamp_corner_rows(kind, n, V, K, seed=71 if kind == "tiny_tau" else 72, dtype=dtype)
    adv = torch.linspace(-1.0, 1.0, n // 4, device=DEV)
    n_valid = sc.count_valid(d["resp_idx"])
    stats = []
    for mode in ("dlogits", "score", "correction"):
        for out_dtype in ("bf16", "f32"):
            say(f"clamp corner {kind} {dtype} {mode}/{out_dtype}")
            out = run_correct(d, adv, n_valid, 1.0, MODES[mode], out_dtype)
            torch.cuda.synchronize()
            assert int(out["status"].item()) == 0
            found = check_rows(f"clamp {kind} {dtype} {mode}/{out_dtype}", d, out,
                               np.arange(n), adv.cpu().numpy(), n, 1.0, MODES[mode],
                               out_dtype, logits_h=z, bf16_stats=stats)
    if kind == "tiny_tau":
        assert all(o["tau"] < 1e-6 and o["S"] < 0.95 for o in found.values())
    else:
        assert all(o["Q_H"] >= 1.0 - 1e-6 for o in found.values())
        assert sum(o["Q_H"] > 1.0 for o in found.values()) >= n // 4
    bf16_bar(stats, f"clamp corner {kind} {dtype}")


@pytest.mark.parametrize("kind", ["tiny_tau", "q_ge_1"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_clamp_corners_two_call(kind, dtype):
    """Both clamp corners through sc_logprobs, then sc_center.  With the
    logits, the second call forms p and log p at H in float64 from them, and
    every output (and the fp32 dLogits row) matches the oracle on the logits.
    Without them (the path after the fused LM-head), its inputs are the
    first call's fp32 log p(a), tail mass and log p at H: those are checked
    against the oracle on the logits, and the centering outputs against the
    oracle's centering from exactly those inputs (sc_center_row), at the same
    bars.  Where rho p_k reaches 1e5 the fp32 logs alone move c_k by many fp32
    steps, so the two are told apart."""
    n, V, K = 32, 4099, 64
    d, z = clamp_corner_rows(kind, n, V, K, seed=73 if kind == "tiny_tau" else 74, dtype=dtype)
    adv = torch.linspace(-1.0, 1.0, n // 4, device=DEV)
    adv_h = adv.cpu().numpy()
    n_valid = sc.count_valid(d["resp_idx"])
    status = [torch.zeros(1, dtype=torch.int32, device=DEV) for _ in range(3)]
    st = sc.logprobs(d["logits"], d["head_ids"], d["sampled"], d["resp_idx"],
                     dev_status=status[0])
    args = (d["head_ids"], d["head_probs"], d["sampled"], d["resp_idx"], adv)
    with_z = {k: v.clone() for k, v in st.items()}
    row_out = torch.empty(n, V, device=DEV)
    sc.center(with_z, *args, n_valid=n_valid, rollout_logp=d["rollout_logp"],
              logits=d["logits"], row_out=row_out, row_mode=O.MODE_DLOGITS,
              dev_status=status[1])
    with_z["row"] = row_out
    no_z = {k: v.clone() for k, v in st.items()}
    sc.center(no_z, *args, n_valid=n_valid, rollout_logp=d["rollout_logp"], vocab=V,
              dev_status=status[2])
    torch.cuda.synchronize()
    assert [int(s.item()) for s in status] == [0, 0, 0]
    say(f"two-call clamp corner {kind} {dtype}, with the logits")
    found = check_rows(f"two-call clamp {kind} {dtype} with logits", d, with_z, np.arange(n),
                       adv_h, n, 1.0, O.MODE_DLOGITS, "f32", logits_h=z)
    assert len(found) == n
    if kind == "tiny_tau":
        assert all(o["tau"] < 1e-6 and o["rho"] > 1e4 for o in found.values())
    say(f"two-call clamp corner {kind} {dtype}, without the logits")
    g = gather(no_z, np.arange(n), None)
    q = host_rows(d["head_probs"], np.arange(n))
    rlp = host_rows(d["rollout_logp"], np.arange(n))
    resp = host_rows(d["resp_idx"], np.arange(n))
    for r in range(n):
        o = found[r]
        gr = {key: val[r] for key, val in g.items()}
        check_row(f"two-call clamp {kind} {dtype} first call row {r}", gr, o, stats_only=True)
        A = float(adv_h[resp[r]])
        lp = gr["head_logp"].astype(np.float64)
        c = O.sc_center_row(float(gr["stats"][1]), float(gr["stats"][2]), lp, q[r],
                            rollout_logp=float(rlp[r]), advantage=A)
        handed = dict(o, logp_a=float(gr["stats"][1]), head_logp=lp, **c)
        check_row(f"two-call clamp {kind} {dtype} centering row {r}", gr, handed, A=A,
                  T=1.0, n_valid=n, rlp=rlp[r])


@pytest.mark.parametrize("T", [1.0, 0.7])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_masked_vocabulary_rows(dtype, T):
    """Rows with a masked (-inf) share of the vocabulary: the statistics
    stream drops those terms from the entropy sum through its recompute path
    (every thread of these rows meets a -inf).  Fused, statistics-only and
    two-call paths, every row against the oracle.  At T = 0.7, log2(e)/T
    rounded to the nearest fp32 leaves a negative remainder, so these rows
    also test how the library splits that scale into an fp32 pair: a -inf
    logit times the pair must stay -inf in every exponent."""
    n, V, K = 24, 50_000, 64
    say(f"masked-vocabulary rows n={n} V={V} K={K} {dtype} T={T}")
    d, z = crafted(n, V, K, seed=9, dtype=dtype)
    rng = np.random.default_rng(10)
    ids = d["head_ids"].cpu().numpy()
    a = d["sampled"].cpu().numpy()
    for r in range(n):
        frac = (0.0, 0.01, 0.4, 0.95)[r % 4]
        mask = rng.random(V) < frac
        mask[ids[r]] = False
        mask[a[r]] = False
        z[r, mask] = -np.inf
    logits = torch.from_numpy(z).to(DEV)
    d["logits"] = logits.to(torch.bfloat16) if dtype == "bf16" else logits
    adv = torch.linspace(-1.0, 1.0, 6, device=DEV)
    n_valid = sc.count_valid(d["resp_idx"])
    out = run_correct(d, adv, n_valid, T, O.MODE_DLOGITS, "bf16")
    s1 = torch.zeros(1, dtype=torch.int32, device=DEV)
    st = sc.logprobs(d["logits"], d["head_ids"], d["sampled"], d["resp_idx"], temperature=T,
                     dev_status=s1)
    torch.cuda.synchronize()
    assert int(out["status"].item()) == 0 and int(s1.item()) == 0
    check_rows(f"masked {dtype} T={T}", d, out, np.arange(n), adv.cpu().numpy(), n, T,
               O.MODE_DLOGITS, "bf16", logits_h=z)
    Tf = float(np.float32(T))
    for r in range(n):
        o = O.sc_row(z[r].astype(np.float64), Tf, ids[r], d["head_probs"][r].cpu().numpy(),
                     a[r])
        g = dict(stats=st["row_stats"][r].cpu().numpy(), idx=st["row_idx"][r].cpu().numpy(),
                 head_logp=st["head_logp"][r].cpu().numpy())
        check_row(f"masked logprobs {dtype} T={T} row {r}", g, o, stats_only=True)
    row_out = torch.empty(n, V, device=DEV)
    s2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    sc.center(st, d["head_ids"], d["head_probs"], d["sampled"], d["resp_idx"], adv,
              temperature=T, n_valid=n_valid, rollout_logp=d["rollout_logp"],
              logits=d["logits"], row_out=row_out, row_mode=O.MODE_DLOGITS, dev_status=s2)
    st["row"] = row_out
    torch.cuda.synchronize()
    assert int(s2.item()) == 0
    check_rows(f"masked two-call {dtype} T={T}", d, st, np.arange(n), adv.cpu().numpy(), n, T,
               O.MODE_DLOGITS, "f32", logits_h=z)


@pytest.mark.parametrize("dtype,K,T", [("f32", 128, 1.0), ("bf16", 1024, 0.6)])
def test_full_vocabulary_fp32_and_k1024(dtype, K, T):
    """Full-vocabulary rows (V = 248,320) on the paths the quick-check bench
    does not take: fp32 logits (4 per 16-byte vector), and K = 1024 recorded
    ids (the row kernels' LDS beyond 64 KB), at another temperature."""
    n, V = 12, synthetic.VOCAB
    say(f"full-vocabulary rows n={n} {dtype} K={K} T={T}")
    d, z = crafted(n, V, K, seed=K + 3, dtype=dtype, scale=2.5)
    adv = torch.tensor([0.8, -1.2, 0.3], device=DEV)
    n_valid = sc.count_valid(d["resp_idx"])
    out = run_correct(d, adv, n_valid, T, O.MODE_DLOGITS, "bf16")
    torch.cuda.synchronize()
    assert int(out["status"].item()) == 0
    check_rows(f"full-V {dtype} K={K}", d, out, np.arange(n), adv.cpu().numpy(), n, T,
               O.MODE_DLOGITS, "bf16", logits_h=z)


def test_many_rows_one_workgroup_each():
    """200,003 short rows: the grid has one workgroup per row, far past
    65,535; the first, the last and sampled rows against the oracle."""
    n, V, K = 200_003, 72, 8
    say(f"many rows n={n} V={V} K={K} bf16")
    d, z = crafted(n, V, K, seed=17, dtype="bf16")
    adv = torch.linspace(-1.5, 1.5, n // 4 + 1, device=DEV)
    n_valid = sc.count_valid(d["resp_idx"])
    out = run_correct(d, adv, n_valid, 1.0, O.MODE_SCORE, "bf16")
    torch.cuda.synchronize()
    assert int(out["status"].item()) == 0
    rows = sample_rows(n, 40, 23, extra=(0, 1, n - 2, n - 1))
    check_rows("many rows", d, out, rows, adv.cpu().numpy(), n, 1.0, O.MODE_SCORE, "bf16",
               logits_h=z[rows])


@pytest.mark.parametrize("V", [1, 2, 7, 8, 9, 17])
def test_tiny_vocabularies(V):
    """Degenerate row lengths: fewer elements than one 16-byte vector, exactly
    one, one plus a partial one; K up to V (K = V makes the tail empty).
    Fused and two-call paths, fp32 and bf16 rows, T = 1 and 0.7.  With V = 1
    the sampled entry e_a - p_a is exactly 0, and the two-call path's is the
    rounding of the log-sum-exp it is handed."""
    for K in sorted({1, min(V, 3), V}):
        for T, out_dtype, two_call in ((1.0, "f32", False), (0.7, "bf16", False),
                                       (0.7, "bf16", True), (1.0, "f32", True)):
            tag = f"tiny V={V} K={K} T={T} {out_dtype} two_call={two_call}"
            say(tag)
            d, z = crafted(16, V, K, seed=V * 7 + K, dtype="f32")
            adv = torch.linspace(-1.0, 1.0, 4, device=DEV)
            n_valid = sc.count_valid(d["resp_idx"])
            if not two_call:
                out = run_correct(d, adv, n_valid, T, O.MODE_SCORE, out_dtype)
            else:
                out = sc.logprobs(d["logits"], d["head_ids"], d["sampled"], d["resp_idx"],
                                  temperature=T)
                row_out = torch.empty(16, V, device=DEV,
                                      dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32)
                out["status"] = torch.zeros(1, dtype=torch.int32, device=DEV)
                sc.center(out, d["head_ids"], d["head_probs"], d["sampled"], d["resp_idx"], adv,
                          temperature=T, n_valid=n_valid, rollout_logp=d["rollout_logp"],
                          logits=d["logits"], row_out=row_out, row_mode=O.MODE_SCORE,
                          dev_status=out["status"])
                out["row"] = row_out
            torch.cuda.synchronize()
            assert int(out["status"].item()) == 0
            check_rows(tag, d, out, np.arange(16), adv.cpu().numpy(), 16, T, O.MODE_SCORE,
                       out_dtype, logits_h=z)


def test_seeded_random_shapes():
    """24 seeded draws of (rows, V, K, dtype, stride, T, row mode, output
    dtype), every row against the oracle."""
    rng = np.random.default_rng(2026)
    stats = []
    for case in range(24):
        V = int(rng.choice([5, 33, 257, 1000, 2049, 4096, 7001, 12289]))
        K = int(min(V, rng.choice([1, 2, 16, 64, 128, 200, 300])))
        n = int(rng.choice([1, 3, 16, 37, 64]))
        dtype = str(rng.choice(["bf16", "f32"]))
        stride = None if rng.random() < 0.6 else V + int(rng.integers(1, 9))
        T = float(rng.choice([1.0, 0.7, 1.3]))
        mode = int(rng.choice([O.MODE_DLOGITS, O.MODE_SCORE, O.MODE_CORRECTION]))
        out_dtype = str(rng.choice(["bf16", "f32"]))
        tag = f"random {case}: n={n} V={V} K={K} {dtype} stride={stride} T={T} mode={mode} out={out_dtype}"
        say(tag)
        d, z = crafted(n, V, K, seed=case, dtype=dtype, stride=stride)
        adv = torch.linspace(-1.2, 1.3, (n + 3) // 4, device=DEV)
        n_valid = sc.count_valid(d["resp_idx"])
        out = run_correct(d, adv, n_valid, T, mode, out_dtype)
        torch.cuda.synchronize()
        assert int(out["status"].item()) == 0
        check_rows(tag, d, out, np.arange(n), adv.cpu().numpy(), n, T, mode, out_dtype,
                   logits_h=z, bf16_stats=stats)
    bf16_bar(stats, "24 random shapes")


@pytest.mark.parametrize("dtype,out_dtype", [("f32", "f32"), ("f32", "bf16"), ("bf16", "f32")])
def test_padding_rows_every_output_layout(dtype, out_dtype):
    """Padding rows (resp_idx = -1) write an all-zero row in every input /
    output dtype pair (16-byte vector zero fill), next to valid rows that
    match the oracle."""
    n, V, K = 24, 4099, 32
    say(f"padding rows {dtype} -> {out_dtype}")
    d, z = crafted(n, V, K, seed=61, dtype=dtype)
    resp = d["resp_idx"].clone()
    resp[1::3] = -1
    d["resp_idx"] = resp
    adv = torch.linspace(-1.0, 1.0, n // 4, device=DEV)
    n_valid = sc.count_valid(d["resp_idx"])
    out = run_correct(d, adv, n_valid, 1.0, O.MODE_DLOGITS, out_dtype)
    torch.cuda.synchronize()
    assert int(out["status"].item()) == 0
    assert int(n_valid.item()) == n - len(range(1, n, 3))
    check_rows(f"padding {dtype}->{out_dtype}", d, out, np.arange(n), adv.cpu().numpy(),
               int(n_valid.item()), 1.0, O.MODE_DLOGITS, out_dtype, logits_h=z)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_argmax_ties_first_index(dtype):
    """Equal maxima planted in one 16-byte vector, in two vectors of one
    thread, across threads and in the partial last vector: the argmax is the
    first of them (the oracle's smallest index of the maximum), from both
    sc_logprobs and sc_correct."""
    say(f"argmax ties dtype={dtype}")
    rng = np.random.default_rng(21)
    n, V, K = 48, 4099, 16
    z = rng.normal(0, 1, (n, V)).astype(np.float32)
    top = 8.0                                    # exact in bf16
    N = 8 if dtype == "bf16" else 4              # elements per 16-byte vector
    patterns = [(5, 6), (3, 3 + N * 256), (3, 3 + N * 384 + N), (N * 7 + 1, N * 7),
                (V - 1, V - 2), (V - 3, 0), (1000, 1001, 1002), (2 * N, 2 * N + N * 300)]
    for r in range(n):
        for p in patterns[r % len(patterns)]:
            z[r, p] = top
    if dtype == "bf16":
        zt = torch.from_numpy(z).to(torch.bfloat16)
        zh = zt.float().numpy()
    else:
        zt = torch.from_numpy(z)
        zh = z
    ids = np.stack([rng.choice(V, K, replace=False) for _ in range(n)]).astype(np.int32)
    q = rng.dirichlet(np.ones(K), n).astype(np.float32) * 0.9
    a = rng.integers(0, V, n).astype(np.int32)
    resp = np.zeros(n, dtype=np.int32)
    d = to_dev(dict(logits=zt, head_ids=ids, head_probs=q, sampled=a, resp_idx=resp))
    st = sc.logprobs(d["logits"], d["head_ids"], d["sampled"], d["resp_idx"])
    adv = torch.ones(1, device=DEV)
    nv = sc.count_valid(d["resp_idx"])
    out = sc.correct(d["logits"], d["head_ids"], d["head_probs"], d["sampled"],
                     d["resp_idx"], adv, n_valid=nv)
    torch.cuda.synchronize()
    got_s = st["row_idx"][:, 0].cpu().numpy()
    got_c = out["row_idx"][:, 0].cpu().numpy()
    for r in range(n):
        o = O.sc_row(zh[r], 1.0, ids[r], q[r], a[r])
        assert o["argmax"] == min(patterns[r % len(patterns)]), r
        assert got_s[r] == o["argmax"] and got_c[r] == o["argmax"], (r, got_s[r], got_c[r], o["argmax"])


def test_flat_rows_k1024_full_vocabulary():
    """Rows whose tail terms are all near their largest: exactly uniform
    logits (every one of the ~8,200 listed elements a tail term of weight
    one, argmax at index 0), uniform with the 1,024 recorded ids in one
    contiguous block, near-flat N(0, 0.01^2), and a two-level row (recorded
    ids one logit above the rest), at V = 248,320, K = 1,024, bf16."""
    n, V, K = 8, synthetic.VOCAB, 1024
    say(f"flat rows n={n} V={V} K={K} bf16")
    d, z = crafted(n, V, K, seed=99, dtype="bf16")
    ids = d["head_ids"].cpu().numpy()
    rng = np.random.default_rng(99)
    z[0:2] = 0.5
    z[2:4] = 0.5
    s0 = int(rng.integers(0, V - K))
    ids[2] = np.arange(s0, s0 + K, dtype=np.int32)
    ids[3] = np.arange(V - K, V, dtype=np.int32)                 # up to the row's end
    z[4:6] = torch.from_numpy(rng.normal(0, 0.01, (2, V)).astype(np.float32)).to(
        torch.bfloat16).float().numpy()
    z[6:8] = 0.0
    z[6, ids[6]] = 1.0
    z[7, ids[7]] = 1.0
    d["head_ids"] = torch.from_numpy(ids).to(DEV)
    d["logits"] = torch.from_numpy(z).to(DEV).to(torch.bfloat16)
    adv = torch.tensor([0.8, -1.2], device=DEV)
    n_valid = sc.count_valid(d["resp_idx"])
    for mode in (O.MODE_DLOGITS, O.MODE_CORRECTION):
        out = run_correct(d, adv, n_valid, 1.0, mode, "bf16")
        torch.cuda.synchronize()
        assert int(out["status"].item()) == 0
        assert out["row_idx"][0, 0].item() == 0 and out["row_idx"][1, 0].item() == 0
        check_rows(f"flat rows mode={mode}", d, out, np.arange(n), adv.cpu().numpy(), n, 1.0,
                   mode, "bf16", logits_h=z)


# Large vocabularies around the full one (whole 256-thread rounds of
# vectors, a ragged tail, one vector more) with a -inf-masked row, the row
# maximum in the last vectors and a flat row; bf16 and fp32 output.
@pytest.mark.parametrize("V", [180224, 180231, 253952, 253960])
def test_large_vocabularies_masked_and_flat_rows(V):
    n, K = 16, 128
    say(f"large vocabulary n={n} V={V} K={K} bf16")
    d, z = crafted(n, V, K, seed=V, dtype="bf16")
    ids = d["head_ids"].cpu().numpy()
    z[3, ::3] = -np.inf                  # masked vocabulary (careful pass-2 values)
    z[3, ids[3]] = 0.25
    z[5, V - 2] = 30.0                   # the row maximum in the last vectors
    z[6, :] = 1.5                        # flat row: argmax 0, equal tail terms
    d["logits"] = torch.from_numpy(z).to(DEV).to(torch.bfloat16)
    adv = torch.tensor([0.8, -1.2, 0.3, 1.1], device=DEV)
    n_valid = sc.count_valid(d["resp_idx"])
    for out_dtype in ("bf16", "f32"):
        out = run_correct(d, adv, n_valid, 1.0, O.MODE_DLOGITS, out_dtype)
        torch.cuda.synchronize()
        assert int(out["status"].item()) == 0
        check_rows(f"large vocabulary V={V} ->{out_dtype}", d, out, np.arange(n),
                   adv.cpu().numpy(), n, 1.0, O.MODE_DLOGITS, out_dtype, logits_h=z)
