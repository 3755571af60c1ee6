"""GPU parity of the fused LM-head statistics (sc_logprobs_lmhead).

Two stages: (1) the fused kernel's GEMM, dumped by sc_lmhead_logits with the
identical accumulation order, against the float64 product of the same bf16
inputs within a rigorous fp32 summation bound; (2) the statistics against the
oracle evaluated on those very logits (so argmax and the gathers are
compared exactly), plus the unfused sc_logprobs on the same logits and the
rest of the correction through sc_center.
"""
import numpy as np
import pytest
import torch

from oracle import sc_oracle as O
import synthetic
from tests.parity import check_row

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from off_policy_logit_amd import sc

DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)


def gen(seed):
    return torch.Generator(device=DEV).manual_seed(seed)


def product_bound(x, w, d):
    """|fp32 sum - exact| <= (d + 16) u sum_k |x_k w_k| for any order of the
    d - 1 additions (bf16 products are exact in fp32)."""
    return (d + 16) * 2.0 ** -24 * (np.abs(x) @ np.abs(w).T)


LOGITS_ABS = 2e-4   # the stated bar on the GEMM's logits against float64


def check_logits(tag, err, x, w, d):
    """Every logit within the stated abs 2e-4 and within the rigorous fp32
    summation bound."""
    tol = product_bound(x, w, d)
    say(f"{tag}: max |err| {float(err.max()):.3e} (bar {LOGITS_ABS})")
    assert float(err.max()) <= LOGITS_ABS, (tag, float(err.max()))
    assert np.all(err <= tol), (tag, float(err.max()), float((err - tol).max()))


@pytest.mark.parametrize("n,V,d,pad", [(600, 4099, 256, 0), (300, 3000, 4096, 0),
                                       (37, 300, 64, 0), (513, 1031, 192, 64),
                                       (1100, 700, 128, 0)])
def test_lmhead_logits_match_float64_product(n, V, d, pad):
    say(f"lmhead logits n={n} V={V} d={d} row padding={pad}")
    w_full = (torch.randn(V, d + pad, generator=gen(1), device=DEV) * 0.05).to(torch.bfloat16)
    x_full = torch.randn(n, d + pad, generator=gen(2), device=DEV).to(torch.bfloat16)
    w, x = w_full[:, :d], x_full[:, :d]
    z = sc.lmhead_logits(x, w)
    torch.cuda.synchronize()
    xh, wh = x.float().cpu().numpy(), w.float().cpu().numpy()
    ref = O.lmhead_logits(xh, wh)
    err = np.abs(z.cpu().numpy().astype(np.float64) - ref)
    check_logits(f"logits n={n} V={V} d={d}", err, xh, wh, d)


def run_lmhead(c, w, resp, T, status=None):
    return sc.logprobs_lmhead(c["hidden"], w, c["head_ids"], c["sampled"], resp,
                              temperature=T, dev_status=status)


def host(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


@pytest.mark.parametrize("T,w_sd", [(1.0, 0.02), (0.7, 0.02), (1.0, 0.25)])
def test_lmhead_stats_match_oracle_on_own_logits(T, w_sd):
    n, V, d = 700, 5003, 512
    say(f"lmhead stats n={n} V={V} d={d} T={T} w_sd={w_sd}")
    w, wr = synthetic.lmhead_weights(DEV, vocab=V, d=d, seed=8, w_sd=w_sd)
    c = synthetic.lmhead_chunk(DEV, wr, n, seed=9, temperature=T)
    resp = torch.zeros(n, dtype=torch.int32, device=DEV)
    resp[5] = -1
    resp[600:610] = -1
    ids = c["head_ids"]
    ids[10, 3] = ids[10, 7]                 # duplicate id
    ids[11, 0] = V                          # id out of range
    c["sampled"][12] = -1                   # sampled id out of range
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = run_lmhead(c, w, resp, T, status)
    z = sc.lmhead_logits(c["hidden"], w)
    torch.cuda.synchronize()
    assert int(status.item()) == (O.DEV_DUP_ID | O.DEV_BAD_ID | O.DEV_BAD_SAMPLED)
    zh, idh, qh, ah, rh = host(z), host(ids), host(c["head_probs"]), host(c["sampled"]), host(resp)
    st, ix, hl = host(out["row_stats"]), host(out["row_idx"]), host(out["head_logp"])
    for r in range(n):
        if rh[r] < 0:
            assert np.all(st[r, [0, 1, 2, 3, 11]] == 0) and list(ix[r]) == [-1, -1]
            assert np.all(hl[r] == 0)
            continue
        o = O.sc_row(zh[r], float(np.float32(T)), idh[r], qh[r], ah[r])
        g = dict(stats=st[r], idx=ix[r], head_logp=hl[r])
        check_row(f"lmhead row {r}", g, o, T=T, stats_only=True)

    # the unfused statistics pass on the same fp32 logits agrees
    say("sc_logprobs on the dumped logits")
    ref = sc.logprobs(z, ids, c["sampled"], resp, temperature=T)
    torch.cuda.synchronize()
    good = np.array([r for r in range(n) if rh[r] >= 0 and r not in (10, 11, 12)])
    np.testing.assert_array_equal(ix[good], host(ref["row_idx"])[good])
    for col, tol in ((0, 1e-5), (1, 1e-5), (2, 1e-6), (3, 1e-6), (11, 2e-5)):
        np.testing.assert_allclose(st[good, col], host(ref["row_stats"])[good, col],
                                   atol=tol, rtol=1e-5)


def test_lmhead_then_center_completes_the_correction():
    n, V, d, T = 384, 2048, 256, 1.0
    say(f"lmhead + sc_center n={n} V={V} d={d}")
    w, wr = synthetic.lmhead_weights(DEV, vocab=V, d=d, seed=10, w_sd=0.1)
    c = synthetic.lmhead_chunk(DEV, wr, n, seed=11, temperature=T)
    resp = torch.arange(n, dtype=torch.int32, device=DEV) // 96       # 4 responses
    rewards = torch.tensor([1.0, 0.0, 0.0, 1.0], device=DEV)
    adv = sc.group_norm(rewards, 4)
    n_valid = sc.count_valid(resp)
    st = run_lmhead(c, w, resp, T)
    sc.center(st, c["head_ids"], c["head_probs"], c["sampled"], resp, adv, temperature=T,
              n_valid=n_valid, rollout_logp=c["rollout_logp"], vocab=V)
    z = sc.lmhead_logits(c["hidden"], w)
    torch.cuda.synchronize()
    zh, adv_h = host(z), host(adv)
    g_all = {key: host(st[key]) for key in ("row_stats", "row_idx", "head_logp", "coef")}
    for r in range(0, n, 5):
        A = float(adv_h[r // 96])
        rlp = float(host(c["rollout_logp"])[r])
        o = O.sc_row(zh[r], float(np.float32(T)), host(c["head_ids"])[r], host(c["head_probs"])[r],
                     int(host(c["sampled"])[r]), rollout_logp=rlp, advantage=A, n_valid=n)
        g = dict(stats=g_all["row_stats"][r], idx=g_all["row_idx"][r],
                 head_logp=g_all["head_logp"][r], coef=g_all["coef"][r])
        check_row(f"lmhead+center row {r}", g, o, A=A, T=T, n_valid=n, rlp=rlp)


def test_lmhead_k_extremes_and_determinism():
    n, V, d = 260, 1500, 128
    for K in (1, 200, 1024):
        say(f"lmhead K={K} n={n} V={V} d={d}, two runs")
        w = (torch.randn(V, d, generator=gen(20 + K), device=DEV) * 0.2).to(torch.bfloat16)
        x = torch.randn(n, d, generator=gen(30 + K), device=DEV).to(torch.bfloat16)
        z = sc.lmhead_logits(x, w)
        ids = torch.argsort(torch.rand(n, V, generator=gen(40 + K), device=DEV), dim=1)[:, :K]
        ids = ids.to(torch.int32).contiguous()
        a = torch.randint(0, V, (n,), generator=gen(50 + K), device=DEV, dtype=torch.int32)
        a[::3] = ids[::3, K // 2]
        c = dict(hidden=x, head_ids=ids, sampled=a)
        o1 = run_lmhead(c, w, None, 1.0)
        o2 = run_lmhead(c, w, None, 1.0)
        torch.cuda.synchronize()
        cols = [sc.STAT[k] for k in ("lse", "logp_a", "tail", "P_H", "entropy")]
        assert torch.equal(o1["row_stats"][:, cols].view(torch.int32),
                           o2["row_stats"][:, cols].view(torch.int32))
        for key in ("row_idx", "head_logp"):
            assert torch.equal(o1[key].view(torch.int32), o2[key].view(torch.int32)), key
        zh, idh, ah = host(z), host(ids), host(a)
        st, ix, hl = host(o1["row_stats"]), host(o1["row_idx"]), host(o1["head_logp"])
        for r in range(0, n, 7):
            o = O.sc_row(zh[r], 1.0, idh[r], np.full(K, 1.0 / V), ah[r])
            check_row(f"K={K} row {r}", dict(stats=st[r], idx=ix[r], head_logp=hl[r]), o,
                      stats_only=True)


def test_lmhead_full_vocab_slice():
    """The bench's launch configuration: 16,384 rows, V = 248,320, d = 4,096."""
    n, V, d = 16_384, synthetic.VOCAB, 4096
    say(f"lmhead full-size slice n={n} V={V} d={d}: generate")
    w, wr = synthetic.lmhead_weights(DEV, vocab=V, d=d, seed=5)
    c = synthetic.lmhead_chunk(DEV, wr, n, seed=6)
    del wr
    torch.cuda.synchronize()
    say("lmhead full-size slice: run")
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = run_lmhead(c, w, None, 1.0, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([rng.choice(n, 20, replace=False), [0, 255, 256, n - 1]]))
    sub = torch.as_tensor(rows, device=DEV)
    z = sc.lmhead_logits(c["hidden"][sub].contiguous(), w)   # same per-element order
    torch.cuda.synchronize()
    zh = host(z)
    st, ix = host(out["row_stats"][sub]), host(out["row_idx"][sub])
    hl = host(out["head_logp"][sub])
    idh, qh, ah = host(c["head_ids"][sub]), host(c["head_probs"][sub]), host(c["sampled"][sub])
    for j, r in enumerate(rows):
        o = O.sc_row(zh[j], 1.0, idh[j], qh[j], ah[j])
        check_row(f"lmhead full row {r}", dict(stats=st[j], idx=ix[j], head_logp=hl[j]), o,
                  stats_only=True)
    # the sampled rows' logits against the float64 product, 16,384 ids at a time
    xh = host(c["hidden"][sub])
    err = np.empty_like(zh, dtype=np.float64)
    for v0 in range(0, V, 16_384):
        wh = host(w[v0:v0 + 16_384])
        err[:, v0:v0 + wh.shape[0]] = np.abs(zh[:, v0:v0 + wh.shape[0]] - O.lmhead_logits(xh, wh))
        check_logits(f"full slice logits ids {v0}+", err[:, v0:v0 + wh.shape[0]], xh, wh, d)


def test_lmhead_more_rows_than_vocabulary():
    """Rows outnumber vocabulary ids: the tile loop's XCD-group order (split
    counts that are not multiples of 8)."""
    n, V, d, T = 2600, 1300, 128, 1.0
    say(f"lmhead stats n={n} V={V} d={d} (more rows than ids)")
    w, wr = synthetic.lmhead_weights(DEV, vocab=V, d=d, seed=21, w_sd=0.1)
    c = synthetic.lmhead_chunk(DEV, wr, n, seed=22, temperature=T)
    out = run_lmhead(c, w, None, T)
    z = sc.lmhead_logits(c["hidden"], w)
    torch.cuda.synchronize()
    zh, idh, qh, ah = host(z), host(c["head_ids"]), host(c["head_probs"]), host(c["sampled"])
    st, ix, hl = host(out["row_stats"]), host(out["row_idx"]), host(out["head_logp"])
    for r in range(0, n, 37):
        o = O.sc_row(zh[r], float(np.float32(T)), idh[r], qh[r], ah[r])
        check_row(f"rows>ids row {r}", dict(stats=st[r], idx=ix[r], head_logp=hl[r]), o,
                  stats_only=True)


def test_lmhead_logits_seeded_random_shapes():
    """12 seeded draws of (rows, V, d, row padding): the GEMM against the
    float64 product (grid order and split count vary with the shape)."""
    rng = np.random.default_rng(404)
    for case in range(12):
        n = int(rng.choice([1, 7, 255, 256, 257, 700, 1300]))
        V = int(rng.choice([1, 63, 256, 257, 999, 2305, 5000]))
        d = int(rng.choice([64, 128, 320, 1024]))
        pad = int(rng.choice([0, 8, 64]))
        say(f"lmhead random {case}: n={n} V={V} d={d} pad={pad}")
        w_full = (torch.randn(V, d + pad, generator=gen(10 + case), device=DEV) * 0.05).to(torch.bfloat16)
        x_full = torch.randn(n, d + pad, generator=gen(50 + case), device=DEV).to(torch.bfloat16)
        w, x = w_full[:, :d], x_full[:, :d]
        z = sc.lmhead_logits(x, w)
        torch.cuda.synchronize()
        xh, wh = x.float().cpu().numpy(), w.float().cpu().numpy()
        err = np.abs(z.cpu().numpy().astype(np.float64) - O.lmhead_logits(xh, wh))
        check_logits(f"random case {case}", err, xh, wh, d)
