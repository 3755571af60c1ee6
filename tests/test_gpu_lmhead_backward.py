"""GPU parity of the LM-head backward: bf16 dLogits recomputed by the MFMA
kernel (sc_lmhead_dlogits) and the gradients dHidden = dZ W, dW = dZ^T X
(sc_lmhead_backward, both products on the library's MFMA loop) against the
float64 oracle on the kernel's own logits.

Tolerances: dLogits rows as the other bf16 rows (one bf16 step of the RNE of
the float64 value, >= 99.99% bit-equal over a test's entries; the kernel takes
lse from the fp32 statistic plus its remainder column).  Gradients: |err| <= 2^-8 sum_k |G||M| elementwise (bf16
rounding of dZ, 2^-9 relative, plus fp32 accumulation over <= 2^14 terms,
2^-10 relative), plus 2^-9 |value| when d_hidden is bf16.
"""
import numpy as np
import pytest
import torch

from oracle import sc_oracle as O
import synthetic
from tests.parity import MIN_BF16_EQUAL, compare_bf16

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from off_policy_logit_amd import sc

DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)


def host(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def forward(n, V, d, T, seed, is_mode=O.IS_NONE, centering=True, w_sd=0.1):
    w, wr = synthetic.lmhead_weights(DEV, vocab=V, d=d, seed=seed, w_sd=w_sd)
    c = synthetic.lmhead_chunk(DEV, wr, n, seed=seed + 1, temperature=T)
    n_resp = 4
    per = (n + n_resp - 1) // n_resp
    resp = (torch.arange(n, device=DEV) // per).to(torch.int32)
    resp[per - 3:per] = -1                       # a few padding rows
    rewards = torch.tensor([1.0, 0.0, 1.0, 0.0], device=DEV)
    adv = sc.group_norm(rewards, 4)
    n_valid = sc.count_valid(resp)
    st = sc.logprobs_lmhead(c["hidden"], w, c["head_ids"], c["sampled"], resp, temperature=T)
    sc.center(st, c["head_ids"], c["head_probs"], c["sampled"], resp, adv, temperature=T,
              n_valid=n_valid, rollout_logp=c["rollout_logp"], vocab=V, is_mode=is_mode,
              is_lo=0.9, is_hi=1.1, centering=centering)
    z = sc.lmhead_logits(c["hidden"], w)
    torch.cuda.synchronize()
    return w, c, resp, adv, n_valid, st, z


def oracle_dlogits(z, T, c, resp, adv, n_valid, rows, is_mode, centering):
    zh, ids, q, a = host(z), host(c["head_ids"]), host(c["head_probs"]), host(c["sampled"])
    rlp, rh, ah = host(c["rollout_logp"]), host(resp), host(adv)
    G = []
    for r in rows:
        if rh[r] < 0:
            G.append(np.zeros(zh.shape[1]))
            continue
        o = O.sc_row(zh[r], float(np.float32(T)), ids[r], q[r], a[r], rollout_logp=rlp[r],
                     advantage=float(ah[rh[r]]), n_valid=n_valid, row_mode=O.MODE_DLOGITS,
                     is_mode=is_mode, is_lo=0.9, is_hi=1.1, centering=centering)
        G.append(o["row"])
    return np.stack(G)


@pytest.mark.parametrize("is_mode,centering,T", [(O.IS_NONE, True, 1.0),
                                                 (O.IS_TIS, True, 0.8),
                                                 (O.IS_MIS, False, 1.0)])
def test_lmhead_dlogits_rows_match_oracle(is_mode, centering, T):
    n, V, d = 384, 2050, 256
    say(f"lmhead dlogits n={n} V={V} d={d} is_mode={is_mode} centering={centering} T={T}")
    w, c, resp, adv, nv, st, z = forward(n, V, d, T, 30, is_mode, centering)
    dz = sc.lmhead_dlogits(c["hidden"], w, st, c["head_ids"], c["head_probs"], c["sampled"],
                           resp, adv, nv, temperature=T, centering=centering)
    torch.cuda.synchronize()
    G = oracle_dlogits(z, T, c, resp, adv, int(nv.item()), range(n), is_mode, centering)
    bits = dz.view(torch.int16).cpu().numpy()
    dist, eq = compare_bf16(bits, G)
    say(f"dlogits bf16: max step distance {dist}, bit-equal {eq:.6f}")
    assert dist <= 1 and eq >= MIN_BF16_EQUAL, (dist, eq)
    pad = host(resp) < 0
    assert np.all(bits[pad] == 0)


@pytest.mark.parametrize("dh_dtype,chunk", [(torch.float32, 128), (torch.bfloat16, 1000)])
def test_lmhead_backward_matches_oracle(dh_dtype, chunk):
    n, V, d, T = 300, 1500, 192, 1.0
    say(f"lmhead backward n={n} V={V} d={d} d_hidden={dh_dtype} chunk={chunk}")
    w, c, resp, adv, nv, st, z = forward(n, V, d, T, 40)
    args = (c["hidden"], w, st, c["head_ids"], c["head_probs"], c["sampled"], resp, adv, nv)
    dh = torch.empty(n, d, dtype=dh_dtype, device=DEV)
    dW = torch.full((V, d), 7.0, device=DEV)           # overwritten, not added to
    sc.lmhead_backward(*args, temperature=T, d_hidden=dh, d_weight=dW, chunk_rows=chunk)
    torch.cuda.synchronize()
    G = oracle_dlogits(z, T, c, resp, adv, int(nv.item()), range(n), O.IS_NONE, True)
    X, W = host(c["hidden"]), host(w)
    rdX, rdW = O.lmhead_backward(X, W, G)
    tol_x = 2.0 ** -8 * (np.abs(G) @ np.abs(W)) + 1e-30
    if dh_dtype == torch.bfloat16:
        tol_x += 2.0 ** -9 * np.abs(rdX)
    tol_w = 2.0 ** -8 * (np.abs(G).T @ np.abs(X)) + 1e-30
    ex = np.abs(host(dh) - rdX) - tol_x
    ew = np.abs(host(dW) - rdW) - tol_w
    assert ex.max() <= 0, float(np.abs(host(dh) - rdX).max())
    assert ew.max() <= 0, float(np.abs(host(dW) - rdW).max())
    # accumulate: a second call adds the same gradient
    say("lmhead backward accumulate")
    sc.lmhead_backward(*args, temperature=T, d_hidden=dh, d_weight=dW, chunk_rows=chunk,
                       accumulate=True)
    torch.cuda.synchronize()
    assert np.all(np.abs(host(dW) - 2 * rdW) - 2 * tol_w <= 0)


def test_lmhead_backward_full_vocab_slice():
    """The bench's launch: 16,384 rows, V = 248,320, d = 4,096, 8,192-row chunks."""
    n, V, d, T = 16_384, synthetic.VOCAB, 4096, 1.0
    say(f"lmhead backward full slice n={n} V={V} d={d}: forward")
    w, c, resp, adv, nv, st, _ = forward(n, V, d, T, 5, w_sd=0.02)
    say("lmhead backward full slice: backward")
    dh = torch.empty(n, d, dtype=torch.bfloat16, device=DEV)
    dW = torch.empty(V, d, device=DEV)
    sc.lmhead_backward(c["hidden"], w, st, c["head_ids"], c["head_probs"], c["sampled"],
                       resp, adv, nv, temperature=T, d_hidden=dh, d_weight=dW, chunk_rows=8192)
    torch.cuda.synchronize()
    # sampled rows of dHidden against the oracle (row by row at full V)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([rng.choice(n, 3, replace=False), [0, n - 1]]))
    sub = torch.as_tensor(rows, device=DEV)
    z = sc.lmhead_logits(c["hidden"][sub].contiguous(), w)
    cs = {k2: v[sub] for k2, v in c.items()}
    G = oracle_dlogits(z, T, cs, resp[sub], adv, int(nv.item()), range(len(rows)),
                       O.IS_NONE, True)
    W = host(w)
    rdX = G @ W
    tol = 2.0 ** -8 * (np.abs(G) @ np.abs(W)) + 2.0 ** -9 * np.abs(rdX) + 1e-30
    assert np.all(np.abs(host(dh[sub]) - rdX) - tol <= 0)
    # dW at any size: every dLogits row sums to zero (sum_v g_v = 1 - S -
    # (1 - S) = 0), so sum_v dW[v] = 0 up to rounding; sum_v |g_v| <=
    # 1 + S + |1 - S| bounds each row's share of the rounding
    colsum = dW.double().sum(0).cpu().numpy()
    sth, rh, ah = host(st["row_stats"]), host(resp), host(adv)
    S = sth[:, sc.STAT["S"]].astype(np.float64)
    A = np.where(rh >= 0, np.abs(ah[np.maximum(rh, 0)]), 0.0)
    l1 = A * sth[:, sc.STAT["weight"]] / (T * int(nv.item())) * (1 + S + np.abs(1 - S))
    l1 = np.where(rh >= 0, l1, 0.0)
    bound = 2.0 ** -8 * (l1 @ np.abs(host(c["hidden"])).astype(np.float64)) + 1e-12
    assert np.all(np.abs(colsum) <= bound), float((np.abs(colsum) / bound).max())
    assert bool(torch.isfinite(dW).all()) and bool(torch.isfinite(dh.float()).all())


def test_lmhead_backward_1024_row_chunks_full_vocab():
    """16 chunks of 1,024 rows at V = 248,320, d = 4,096 against the bench's
    8,192-row chunks on the same inputs: dHidden bit-identical (each row's
    product runs over the same vocabulary tiles in the same order, and both
    chunk sizes are whole 256-row tiles), dW within the rounding bound of
    the two accumulation orders, and sampled dHidden rows against the
    oracle."""
    n, V, d, T = 16_384, synthetic.VOCAB, 4096, 1.0
    say(f"lmhead backward 1024-row chunks n={n} V={V} d={d}: forward")
    w, c, resp, adv, nv, st, _ = forward(n, V, d, T, 7, w_sd=0.02)
    args = (c["hidden"], w, st, c["head_ids"], c["head_probs"], c["sampled"], resp, adv, nv)
    out = {}
    for chunk in (8192, 1024):
        say(f"lmhead backward 1024-row chunks: backward with chunk_rows={chunk}")
        dh = torch.empty(n, d, dtype=torch.float32, device=DEV)
        dW = torch.empty(V, d, device=DEV)
        sc.lmhead_backward(*args, temperature=T, d_hidden=dh, d_weight=dW, chunk_rows=chunk)
        torch.cuda.synchronize()
        out[chunk] = (dh, dW)
    assert torch.equal(out[1024][0].view(torch.int32), out[8192][0].view(torch.int32))
    dW1, dW8 = out[1024][1].double(), out[8192][1].double()
    # each dW entry is a sum over the 16,384 rows of bf16 dZ x X products in
    # fp32: both orders lie within 2^-8 sum |dZ||X| of the exact value
    rng = np.random.default_rng(5)
    vs = torch.as_tensor(np.unique(rng.choice(V, 64, replace=False)), device=DEV)
    dzt = sc.lmhead_dlogits(c["hidden"], w, st, c["head_ids"], c["head_probs"], c["sampled"],
                            resp, adv, nv, temperature=T)
    g = dzt[:, vs].double()                               # [n, 64]
    del dzt
    bound = 2.0 ** -7 * (g.abs().T @ c["hidden"].double().abs())
    assert bool(((dW1[vs] - dW8[vs]).abs() <= bound).all())
    rows = np.unique(np.concatenate([rng.choice(n, 3, replace=False), [0, 1023, 1024, n - 1]]))
    sub = torch.as_tensor(rows, device=DEV)
    z = sc.lmhead_logits(c["hidden"][sub].contiguous(), w)
    cs = {k2: v[sub] for k2, v in c.items()}
    G = oracle_dlogits(z, T, cs, resp[sub], adv, int(nv.item()), range(len(rows)),
                       O.IS_NONE, True)
    W = host(w)
    rdX = G @ W
    tol = 2.0 ** -8 * (np.abs(G) @ np.abs(W)) + 1e-30
    assert np.all(np.abs(host(out[1024][0][sub]) - rdX) - tol <= 0)
