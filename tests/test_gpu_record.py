"""GPU parity of the rollout-side record (sc_record) against the oracle.

Candidate ids must match exactly (the selection is a decision on the input
values; ties go to the lower id); probabilities within abs 1e-6 + rel 4e-6
(one fp32 exp2 of an fp32 fma after an fp32 log-sum-exp, as in the trainer
statistics); the sampled log-probability within abs 1e-5, the bar for
log-probabilities (the kernel forms it in float64 from the exact logit
difference, and its fp32 value is then within half an ulp).
"""
import numpy as np
import pytest
import torch

from oracle import sc_oracle as O
import synthetic

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from off_policy_logit_amd import sc

DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)


def host(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def check(tag, z_rows, T, k, sampled, out, rows=None):
    ids, probs = host(out["head_ids"]), host(out["head_probs"])
    lp = host(out["sampled_logp"]) if out["sampled_logp"] is not None else None
    rows = range(z_rows.shape[0]) if rows is None else rows
    for j, r in enumerate(rows):
        a = None if sampled is None else int(sampled[j])
        o = O.record_topk(z_rows[j], T, k, sampled=a)
        if o["flags"]:
            assert np.all(ids[r] == -1) and np.all(np.isnan(probs[r])), (tag, r)
            continue
        np.testing.assert_array_equal(ids[r], o["head_ids"], err_msg=f"{tag} row {r}")
        err = np.abs(probs[r] - o["head_probs"]) - (1e-6 + 4e-6 * o["head_probs"])
        assert err.max() <= 0, (tag, r, float(np.abs(probs[r] - o["head_probs"]).max()))
        if lp is not None:
            tol = max(1e-5, float(np.spacing(np.float32(abs(o["sampled_logp"])))))
            assert abs(lp[r] - o["sampled_logp"]) <= tol, (tag, r, lp[r], o["sampled_logp"])


@pytest.mark.parametrize("T", [1.0, 0.7])
@pytest.mark.parametrize("k", [128, 1, 300])
def test_record_tiny_every_row(T, k):
    say(f"record tiny 256 x 4096 fp32 T={T} k={k}")
    h = synthetic.tiny(seed=5, temperature=T)
    z = torch.from_numpy(h["logits"]).to(DEV)
    a = torch.from_numpy(h["sampled"]).to(DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = sc.record(z, k, sampled=a, temperature=T, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    check(f"tiny T={T} k={k}", h["logits"], T, k, h["sampled"], out)


def test_record_ties_masks_ragged_and_strided():
    V = 2003
    rows = []
    rng = np.random.default_rng(7)
    rows.append(np.zeros(V))                                   # all equal: fallback path
    x = np.round(rng.normal(0, 1, V) * 4) / 4                  # heavy ties everywhere
    rows.append(x)
    x = np.full(V, -1.0); x[rng.choice(V, 500, replace=False)] = 2.0   # tie group > k
    rows.append(x)
    x = rng.normal(0, 1, V); x[rng.choice(V, 1900, replace=False)] = -np.inf  # masked
    rows.append(x)
    x = np.full(V, -np.inf); x[[3, 1000, 2002]] = [1.0, 1.0, 0.5]    # fewer finite than k
    rows.append(x)
    x = np.sort(rng.normal(0, 3, V))                           # sorted: top-k in one run
    rows.append(x)
    rows.append(x[::-1].copy())
    x = rng.normal(0, 3, V); x[5] = -0.0; x[6] = 0.0           # signed zeros tie
    rows.append(x)
    z = np.stack(rows).astype(np.float32)
    n = z.shape[0]
    sampled = rng.integers(0, V, n).astype(np.int32)
    sampled[4] = 1000
    for dtype in (torch.float32, torch.bfloat16):
        for stride in (V, V + 5):
            for k in (1, 64, 512):
                say(f"record crafted {dtype} stride={stride} k={k}")
                buf = torch.zeros(n, stride, dtype=dtype, device=DEV)
                buf[:, :V] = torch.from_numpy(z).to(DEV).to(dtype)
                zt = buf[:, :V]
                zh = host(zt)
                a = torch.from_numpy(sampled).to(DEV)
                out = sc.record(zt, k, sampled=a)
                torch.cuda.synchronize()
                check(f"crafted {dtype} stride={stride} k={k}", zh, 1.0, k, sampled, out)


def test_record_flags():
    V = 300
    z = torch.randn(4, V, device=DEV)
    z[1, 17] = float("nan")
    z[2] = float("-inf")
    a = torch.tensor([5, 6, 7, V], dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    say("record flags")
    out = sc.record(z, 10, sampled=a, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == (O.DEV_NONFINITE | O.DEV_BAD_SAMPLED)
    check("flags", host(z), 1.0, 10, host(a), out)
    ids = host(out["head_ids"])
    assert np.all(ids[[1, 2, 3]] == -1) and np.all(ids[0] >= 0)


@pytest.fixture(scope="module")
def quick():
    say("generate quick-check workload 8192 x 248320 bf16")
    d = synthetic.quick_check(DEV)
    torch.cuda.synchronize()
    return d


def test_record_full_vocab_rows(quick):
    """The bench's launch: 8,192 rows of bf16 logits at V = 248,320, k = 128."""
    d = quick
    say("record quick-check 8192 x 248320 bf16, k=128")
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = sc.record(d["logits"], 128, sampled=d["sampled"], dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    rng = np.random.default_rng(14)
    rows = np.unique(np.concatenate([rng.choice(8192, 24, replace=False), [0, 8191]]))
    sub = torch.as_tensor(rows, device=DEV)
    check("quick-check", host(d["logits"][sub]), 1.0, 128, host(d["sampled"][sub]), out,
          rows=rows)
    # every row: the recorded ids are distinct, in range, by non-increasing logit
    ids = out["head_ids"].long()
    zs = torch.gather(d["logits"].float(), 1, ids)
    assert bool((zs[:, 1:] <= zs[:, :-1]).all())
    assert int(ids.min()) >= 0 and int(ids.max()) < synthetic.VOCAB
    srt = torch.sort(ids, dim=1).values
    assert bool((srt[:, 1:] != srt[:, :-1]).all())


@pytest.mark.parametrize("sigma", [0.1])
def test_record_stress_rows(sigma):
    say(f"record stress sigma={sigma} chunk (peaked / flat / mixed rows)")
    d = synthetic.stress_chunk(DEV, 0, sigma, chunk_rows=2048)
    out = sc.record(d["logits"], 128, sampled=d["sampled"])
    torch.cuda.synchronize()
    rows = np.arange(0, 2048, 97)
    sub = torch.as_tensor(rows, device=DEV)
    check(f"stress {sigma}", host(d["logits"][sub]), 1.0, 128, host(d["sampled"][sub]), out,
          rows=rows)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("k", [128, 700])
def test_record_sign_and_magnitude_regimes(dtype, k):
    """Rows whose top-k and maximum sit far apart in key order (all positive,
    all negative, tiny magnitudes across many exponents, wide spread, mixed
    large and tiny), over enough tiles that the running bound is re-read
    several times; V ragged (not a multiple of 8)."""
    V = 70_001
    rng = np.random.default_rng(21)
    rows = []
    for _ in range(3):
        rows.append(rng.normal(0, 3, V) + 40.0)
        rows.append(rng.normal(0, 3, V) - 40.0)
        rows.append(rng.normal(0, 1, V) * 1e-3)
        rows.append(rng.normal(0, 30, V))
        x = rng.normal(0, 1, V) * 1e-4
        big = rng.choice(V, 400, replace=False)
        x[big] = rng.normal(5, 2, 400)
        rows.append(x)
    z = np.stack(rows).astype(np.float32)
    n = z.shape[0]
    sampled = rng.integers(0, V, n).astype(np.int32)
    say(f"record regimes {n} x {V} {dtype} k={k}")
    zt = torch.from_numpy(z).to(DEV).to(dtype)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = sc.record(zt, k, sampled=torch.from_numpy(sampled).to(DEV), dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    check(f"regimes {dtype} k={k}", host(zt), 1.0, k, sampled, out)


def test_record_many_rows():
    """200,003 short rows (one workgroup each, a grid far past 65,535)."""
    n, V, k = 200_003, 300, 16
    rng = np.random.default_rng(31)
    z = rng.normal(0, 2, (n, V)).astype(np.float32)
    sampled = rng.integers(0, V, n).astype(np.int32)
    say(f"record many rows n={n} V={V} k={k}")
    zt = torch.from_numpy(z).to(DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = sc.record(zt, k, sampled=torch.from_numpy(sampled).to(DEV), dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    rows = np.unique(np.concatenate([rng.choice(n, 40, replace=False), [0, 1, n - 2, n - 1]]))
    sub = torch.as_tensor(rows, device=DEV)
    check("many rows", z[rows], 1.0, k, sampled[rows], out, rows=rows)


@pytest.mark.parametrize("V", [1, 2, 7, 8, 9, 17])
def test_record_tiny_vocabularies(V):
    rng = np.random.default_rng(V)
    z = rng.normal(0, 2, (16, V)).astype(np.float32)
    sampled = rng.integers(0, V, 16).astype(np.int32)
    for k in sorted({1, min(V, 3), V}):
        say(f"record tiny vocabulary V={V} k={k}")
        out = sc.record(torch.from_numpy(z).to(DEV), k,
                        sampled=torch.from_numpy(sampled).to(DEV))
        torch.cuda.synchronize()
        check(f"tiny V={V} k={k}", z, 1.0, k, sampled, out)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_record_flat_rows_full_vocabulary(dtype):
    """Near-flat rows over the full 248,320-id vocabulary (every logit 0.25,
    one in fifty 1.0, padded rows): each thread of a row sums ~1,000
    comparable terms, the case that asks most of the row sum's precision.
    Ids exact (many ties: the exact fallback), probabilities and the sampled
    log-probability at their bars, for k = 2 and k = 128."""
    V, n = 248_320, 4
    rng = np.random.default_rng(91)
    z = np.full((n, V), 0.25, np.float32)
    for r in range(n):
        z[r, rng.integers(0, V, V // 50)] = 1.0
    sampled = rng.integers(0, V, n).astype(np.int32)
    buf = torch.zeros(n, V + 3, dtype=dtype, device=DEV)
    buf[:, :V] = torch.from_numpy(z).to(DEV).to(dtype)
    zt = buf[:, :V]
    for k in (2, 128):
        say(f"record flat rows V={V} k={k} {dtype}")
        out = sc.record(zt, k, sampled=torch.from_numpy(sampled).to(DEV))
        torch.cuda.synchronize()
        check(f"flat V={V} k={k}", host(zt), 1.0, k, sampled, out)


def test_record_seeded_random_shapes():
    """24 seeded draws of (rows, V, k, dtype, stride, T), every row against
    the oracle."""
    rng = np.random.default_rng(2027)
    for case in range(24):
        V = int(rng.choice([5, 33, 257, 1000, 2049, 4096, 7001, 12289]))
        k = int(min(V, rng.choice([1, 8, 128, 256, 300])))
        n = int(rng.choice([1, 3, 16, 37]))
        dtype = torch.bfloat16 if rng.random() < 0.5 else torch.float32
        stride = V if rng.random() < 0.6 else V + int(rng.integers(1, 9))
        T = float(rng.choice([1.0, 0.7, 1.3]))
        say(f"record random {case}: n={n} V={V} k={k} {dtype} stride={stride} T={T}")
        z = rng.normal(0, float(rng.choice([0.5, 2.0, 6.0])), (n, V)).astype(np.float32)
        buf = torch.zeros(n, stride, dtype=dtype, device=DEV)
        buf[:, :V] = torch.from_numpy(z).to(DEV).to(dtype)
        zt = buf[:, :V]
        sampled = rng.integers(0, V, n).astype(np.int32)
        out = sc.record(zt, k, sampled=torch.from_numpy(sampled).to(DEV), temperature=T)
        torch.cuda.synchronize()
        check(f"random {case}", host(zt), T, k, sampled, out)
