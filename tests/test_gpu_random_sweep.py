"""Seeded random sweeps of the three row paths, the recorder and the fused
LM-head against the oracle: many small shapes drawn over every axis at once
(vocabulary from 1 id up, K up to V, fp32 and bf16 logits, strides,
temperatures whose fp32 scale split differs, logit scales 0.1-20, masked
logits, every row mode, output dtype and weighting, the two-call path with
and without the logits).  Each case is checked at the parity bars of
tests/parity.py; the call without logits is checked in two parts (the first
call's outputs against the oracle on the logits, the centering against the
oracle's centering from the statistics it was handed).
"""
import numpy as np
import pytest
import torch

from oracle import sc_oracle as O
from tests.parity import bf16_bar, check_row
from tests.test_gpu_parity import crafted, check_rows, gather, run_correct
from tests.test_gpu_record import check as check_record, host

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from off_policy_logit_amd import sc

DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)


WEIGHTINGS = [dict(), dict(is_mode=O.IS_TIS, is_lo=0.8, is_hi=1.25, centering=True),
              dict(is_mode=O.IS_MIS, is_lo=0.8, is_hi=1.25, centering=True),
              dict(is_mode=O.IS_MIS, is_lo=0.8, is_hi=1.25, centering=False),
              dict(is_mode=O.IS_NONE, centering=False)]


def _masked(d, z, rng, stride, dtype):
    """-inf on a third of the ids that are neither recorded nor sampled."""
    n, V = z.shape
    ids = d["head_ids"].cpu().numpy()
    a = d["sampled"].cpu().numpy()
    keep = np.zeros((n, V), bool)
    keep[np.arange(n)[:, None], ids] = True
    keep[np.arange(n), a] = True
    z = z.copy()
    z[(rng.random((n, V)) < 0.33) & ~keep] = -np.inf
    buf = torch.zeros(n, stride or V, dtype=torch.float32)
    buf[:, :V] = torch.from_numpy(z)
    t = buf.to(DEV)
    d["logits"] = (t.to(torch.bfloat16) if dtype == "bf16" else t)[:, :V]
    return z


def test_rows_random_sweep():
    """200 seeded cases through sc_correct, or sc_logprobs then sc_center."""
    stats, counts = [], dict(fused=0, two_call=0, no_logits=0, rows=0)
    for case in range(200):
        rng = np.random.default_rng(40_000 + case)
        V = int(rng.choice([1, 2, 7, 8, 9, 17, 100, 257, 1000, 2049, 4096, 9001]))
        K = int(min(V, rng.choice([1, 2, 3, 16, 64, 128, 129, 300, 1024])))
        n = int(rng.choice([1, 2, 5, 16]))
        dtype = str(rng.choice(["bf16", "f32"]))
        stride = None if rng.random() < 0.6 else V + int(rng.integers(1, 9))
        T = float(rng.choice([0.5, 0.7, 0.8, 1.0, 1.3, 2.0]))
        mode = int(rng.choice([O.MODE_DLOGITS, O.MODE_SCORE, O.MODE_CORRECTION]))
        out_dtype = [None, "bf16", "f32"][int(rng.integers(0, 3))]
        scale = float(rng.choice([0.1, 1.0, 2.0, 5.0, 20.0]))
        wkw = WEIGHTINGS[int(rng.integers(0, len(WEIGHTINGS)))]
        mask = rng.random() < 0.25
        path = str(rng.choice(["fused", "two_call", "no_logits"]))
        if path == "no_logits":
            out_dtype = None
        tag = (f"rows {case}: n={n} V={V} K={K} {dtype} stride={stride} T={T} mode={mode} "
               f"out={out_dtype} scale={scale} w={wkw} mask={mask} {path}")
        say(tag)
        d, z = crafted(n, V, K, seed=40_000 + case, dtype=dtype, stride=stride, scale=scale)
        if mask:
            z = _masked(d, z, rng, stride, dtype)
        adv = torch.linspace(-1.2, 1.3, (n + 3) // 4, device=DEV)
        n_valid = sc.count_valid(d["resp_idx"])
        if path == "fused":
            out = run_correct(d, adv, n_valid, T, mode, out_dtype, **wkw)
        else:
            out = sc.logprobs(d["logits"], d["head_ids"], d["sampled"], d["resp_idx"],
                              temperature=T)
            row_out = None
            if out_dtype is not None:
                row_out = torch.empty(n, V, device=DEV, dtype=torch.bfloat16
                                      if out_dtype == "bf16" else torch.float32)
            out["status"] = torch.zeros(1, dtype=torch.int32, device=DEV)
            sc.center(out, d["head_ids"], d["head_probs"], d["sampled"], d["resp_idx"], adv,
                      temperature=T, n_valid=n_valid, rollout_logp=d["rollout_logp"],
                      logits=d["logits"] if path == "two_call" else None, row_out=row_out,
                      row_mode=mode, dev_status=out["status"], vocab=V, **wkw)
            out["row"] = row_out
        torch.cuda.synchronize()
        assert int(out["status"].item()) == 0, tag
        counts[path] += 1
        counts["rows"] += n
        if path != "no_logits":
            check_rows(tag, d, out, np.arange(n), adv.cpu().numpy(), n, T, mode, out_dtype,
                       logits_h=z, bf16_stats=stats, **wkw)
            continue
        g = gather(out, np.arange(n), None)
        ids, q = d["head_ids"].cpu().numpy(), d["head_probs"].cpu().numpy()
        a, rlp = d["sampled"].cpu().numpy(), d["rollout_logp"].cpu().numpy()
        resp, adv_h = d["resp_idx"].cpu().numpy(), adv.cpu().numpy()
        Tf = float(np.float32(T))
        for r in range(n):
            A = float(adv_h[resp[r]])
            o = O.sc_row(z[r].astype(np.float64), Tf, ids[r], q[r], int(a[r]),
                         rollout_logp=float(rlp[r]), advantage=A, n_valid=n, row_mode=mode,
                         **wkw)
            o.pop("row")
            gr = {key: val[r] for key, val in g.items()}
            check_row(f"{tag} first call row {r}", gr, o, stats_only=True)
            lp = gr["head_logp"].astype(np.float64)
            c = O.sc_center_row(float(gr["stats"][1]), float(gr["stats"][2]), lp, q[r],
                                rollout_logp=float(rlp[r]), advantage=A, **wkw)
            handed = dict(o, logp_a=float(gr["stats"][1]), head_logp=lp, **c)
            check_row(f"{tag} centering row {r}", gr, handed, A=A, T=Tf, n_valid=n, mode=mode,
                      rlp=rlp[r], **wkw)
    say(f"rows sweep: {counts}")
    assert min(counts["fused"], counts["two_call"], counts["no_logits"]) >= 40
    bf16_bar(stats, "rows sweep")


def test_record_random_sweep():
    """150 seeded cases through sc_record: normal, tied, masked, near-flat
    and spiked rows."""
    rows = 0
    for case in range(150):
        rng = np.random.default_rng(50_000 + case)
        V = int(rng.choice([1, 2, 7, 8, 9, 17, 100, 257, 1000, 2049, 4096, 12289, 33000]))
        k = int(min(V, rng.choice([1, 2, 8, 128, 129, 256, 257, 700, 1024])))
        n = int(rng.choice([1, 3, 16]))
        dtype = torch.bfloat16 if rng.random() < 0.5 else torch.float32
        stride = V if rng.random() < 0.6 else V + int(rng.integers(1, 9))
        T = float(rng.choice([0.5, 0.7, 1.0, 1.3]))
        kind = int(rng.integers(0, 6))
        scale = float(rng.choice([0.01, 0.5, 2.0, 6.0, 30.0]))
        z = rng.normal(float(rng.choice([0.0, -3.0, 2.0])), scale, (n, V)).astype(np.float32)
        if kind == 1:
            z = np.round(z * 4) / 4
        elif kind == 2:
            z[rng.random((n, V)) < 0.4] = -np.inf
        elif kind == 3:
            z[:, :] = 0.25
            z[:, rng.integers(0, V, max(1, V // 50))] = 1.0
        elif kind == 4:
            z = np.where(rng.random((n, V)) < 0.01, z + 8.0, z).astype(np.float32)
        tag = f"record {case}: n={n} V={V} k={k} {dtype} stride={stride} T={T} kind={kind}"
        say(tag)
        buf = torch.zeros(n, stride, dtype=dtype, device=DEV)
        buf[:, :V] = torch.from_numpy(z).to(DEV).to(dtype)
        zt = buf[:, :V]
        zh = host(zt)
        sampled = np.array([int(rng.choice(np.flatnonzero(np.isfinite(zh[r]))))
                            if np.isfinite(zh[r]).any() else 0 for r in range(n)], np.int32)
        out = sc.record(zt, k, sampled=torch.from_numpy(sampled).to(DEV), temperature=T)
        torch.cuda.synchronize()
        check_record(tag, zh, T, k, sampled, out)
        rows += n
    say(f"record sweep: 150 cases, {rows} rows")


def test_lmhead_random_sweep():
    """40 seeded cases through sc_logprobs_lmhead, a third with sc_center
    after it, against the oracle on the GEMM's own logits."""
    rows = 0
    for case in range(40):
        rng = np.random.default_rng(60_000 + case)
        V = int(rng.choice([1, 2, 31, 255, 256, 257, 1000, 4099]))
        K = int(min(V, rng.choice([1, 2, 64, 128, 129, 300])))
        n = int(rng.choice([1, 7, 64, 255, 256, 257]))
        d = int(rng.choice([64, 128, 192, 512]))
        T = float(rng.choice([0.5, 0.7, 1.0, 1.3]))
        w_sd = float(rng.choice([0.01, 0.05, 0.2, 0.6]))
        center = rng.random() < 0.35
        tag = f"lmhead {case}: n={n} V={V} K={K} d={d} T={T} w_sd={w_sd} center={center}"
        say(tag)
        g = torch.Generator(device=DEV).manual_seed(60_000 + case)
        w = (torch.randn(V, d, generator=g, device=DEV) * w_sd).to(torch.bfloat16)
        x = torch.randn(n, d, generator=g, device=DEV).to(torch.bfloat16)
        ids = np.stack([rng.choice(V, K, replace=False) for _ in range(n)]).astype(np.int32)
        q = (rng.dirichlet(np.ones(K), n) * rng.uniform(0.2, 0.999, (n, 1))).astype(np.float32)
        a = rng.integers(0, V, n).astype(np.int32)
        a[:n // 2] = ids[np.arange(n // 2), rng.integers(0, K, n // 2)]
        rlp = np.log(rng.uniform(0.01, 1.0, n)).astype(np.float32)
        resp = (np.arange(n) // 4).astype(np.int32)
        resp[rng.random(n) < 0.1] = -1
        tid, ta, tresp = (torch.from_numpy(v).to(DEV) for v in (ids, a, resp))
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        st = sc.logprobs_lmhead(x, w, tid, ta, tresp, temperature=T, dev_status=status)
        z = sc.lmhead_logits(x, w)
        adv_h = None
        if center:
            adv = torch.linspace(-1.0, 1.0, max(1, int(resp.max()) + 1), device=DEV)
            sc.center(st, tid, torch.from_numpy(q).to(DEV), ta, tresp, adv, temperature=T,
                      n_valid=sc.count_valid(tresp), rollout_logp=torch.from_numpy(rlp).to(DEV),
                      vocab=V, dev_status=status)
            adv_h = adv.cpu().numpy()
        torch.cuda.synchronize()
        assert int(status.item()) == 0, tag
        zh = z.cpu().numpy()
        stats, idx, hl = (st[key].cpu().numpy() for key in ("row_stats", "row_idx", "head_logp"))
        coef = st["coef"].cpu().numpy() if center else None
        Tf = float(np.float32(T))
        for r in range(n):
            if resp[r] < 0:
                assert list(idx[r]) == [-1, -1], (tag, r)
                continue
            A = float(adv_h[resp[r]]) if center else 1.0
            o = O.sc_row(zh[r].astype(np.float64), Tf, ids[r], q[r], int(a[r]),
                         rollout_logp=float(rlp[r]), advantage=A)
            gr = dict(stats=stats[r], idx=idx[r], head_logp=hl[r])
            check_row(f"{tag} row {r}", gr, o, stats_only=True)
            if center:
                lp = hl[r].astype(np.float64)
                c = O.sc_center_row(float(stats[r][1]), float(stats[r][2]), lp, q[r],
                                    rollout_logp=float(rlp[r]), advantage=A)
                gr["coef"] = coef[r]
                check_row(f"{tag} centering row {r}", gr,
                          dict(o, logp_a=float(stats[r][1]), head_logp=lp, **c), A=A, T=Tf,
                          rlp=rlp[r])
            rows += 1
    say(f"lmhead sweep: 40 cases, {rows} rows")
