"""The library's C ABI and its row, LM-head and recorder kernels on the CPU, under
AddressSanitizer and UndefinedBehaviorSanitizer (tests/host: the kernels are
compiled for the host against an emulated device environment in which every
GPU thread is a fiber, wave operations and barriers switch fibers, and
buffer-resource accesses are bounds checked).

* argument checks and workspace-size arithmetic at the extremes;
* seeded random shapes through sc_logprobs, sc_correct and sc_center (data
  errors, -inf / NaN logits, ragged vectors, strided rows), sc_correct's
  outputs on every row compared with the oracle at the GPU tests' bar;
* sc_record (the rollout-side top-k) on seeded random shapes, ties, equal
  rows that take the exact fallback, masks and K past 256: ids exact,
  probabilities and the sampled log-probability at the GPU tests' bars;
* the LM-head entry points on one small ragged problem (two row tiles, two
  vocabulary tiles, a three-chunk backward), their outputs compared with the
  oracle: logits with the fp32 summation bound, statistics at the row
  kernels' tolerances, dLogits at the bf16 bar, dHidden and dW with the
  backward's tolerance.  This also pins the emulated MFMA's operand layout.

A sanitizer finding, an out-of-range store, a barrier deadlock or a failed
entry point ends the harness with a non-zero status.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

from oracle import sc_oracle as O
import torch

from off_policy_logit_amd.sc import SC_BF16
from tests.parity import MIN_BF16_EQUAL, bf16_bar, check_row, compare_bf16

HOST = os.path.join(os.path.dirname(os.path.abspath(__file__)), "host")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:detect_stack_use_after_return=0",
           UBSAN_OPTIONS="print_stacktrace=1")


@pytest.fixture(scope="module")
def harness():
    sys.path.insert(0, HOST)
    try:
        import build as host_build
        return host_build.build()
    finally:
        sys.path.remove(HOST)


def run(exe, *args):
    res = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, env=ENV,
                         timeout=900)
    tail = (res.stdout[-2000:] + res.stderr[-4000:])
    assert res.returncode == 0 and "HARNESS OK" in res.stdout, tail
    return res.stdout


def test_abi_checks_under_sanitizers(harness):
    out = run(harness, "abi")
    assert "0 failures" in out


def read_rows(path):
    """The cases `harness rows ... OUT` recorded: sc_correct's inputs and
    outputs per case."""
    b = open(path, "rb").read()
    o = 0

    def take(dt, n):
        nonlocal o
        a = np.frombuffer(b, dt, n, o)
        o += a.nbytes
        return a
    cases = []
    while o < len(b):
        n, V, K, stride, dtype, out_dtype, mode = (int(v) for v in take(np.int32, 7))
        c = dict(n=n, V=V, K=K, dtype=dtype, out_dtype=out_dtype, mode=mode,
                 T=float(take(np.float32, 1)[0]))
        z = take(np.float32, n * stride).reshape(n, stride)[:, :V]
        if dtype == SC_BF16:   # the kernel read the logits rounded to bf16 (RNE)
            z = torch.from_numpy(z.copy()).to(torch.bfloat16).float().numpy()
        c["z"] = z.astype(np.float64)
        c["ids"] = take(np.int32, n * K).reshape(n, K)
        c["q"] = take(np.float32, n * K).reshape(n, K)
        c["sampled"] = take(np.int32, n)
        c["resp"] = take(np.int32, n)
        c["rlp"] = take(np.float32, n)
        c["adv"] = take(np.float32, n)
        c["n_valid"] = int(take(np.int64, 1)[0])
        c["stats"] = take(np.float32, n * 16).reshape(n, 16)
        c["idx"] = take(np.int32, n * 2).reshape(n, 2)
        c["hl"] = take(np.float32, n * K).reshape(n, K)
        c["coef"] = take(np.float32, n * K).reshape(n, K)
        if out_dtype == SC_BF16:
            c["row"] = take(np.uint16, n * stride).reshape(n, stride)[:, :V]
        else:
            c["row"] = take(np.float32, n * stride).reshape(n, stride)[:, :V]
        cases.append(c)
    return cases


def test_row_kernels_random_shapes_under_sanitizers(harness, tmp_path):
    """Bounds and sanitizers on every entry point, and sc_correct's outputs
    (statistics, coefficients, the row in every mode and output type) on
    every row against the oracle at the GPU tests' bar."""
    path = tmp_path / "rows.bin"
    out = run(harness, "rows", 32, 3, path)
    assert out.count("rows case") == 32
    cases = read_rows(path)
    assert len(cases) == 32
    modes = {0: O.MODE_DLOGITS, 1: O.MODE_SCORE, 2: O.MODE_CORRECTION}
    bf, checked = [], 0
    for ci, c in enumerate(cases):
        row_dtype = "bf16" if c["out_dtype"] == SC_BF16 else "f32"
        for p in range(c["n"]):
            g = dict(stats=c["stats"][p], idx=c["idx"][p], head_logp=c["hl"][p],
                     coef=c["coef"][p], row=c["row"][p])
            if c["resp"][p] < 0:
                assert np.all(g["stats"][:15] == 0) and list(g["idx"]) == [-1, -1]
                assert np.all(g["row"] == 0)
                continue
            A = float(c["adv"][c["resp"][p]])
            o = O.sc_row(c["z"][p], c["T"], c["ids"][p], c["q"][p], int(c["sampled"][p]),
                         rollout_logp=float(c["rlp"][p]), advantage=A,
                         n_valid=c["n_valid"], row_mode=modes[c["mode"]])
            check_row(f"emulated rows case {ci} row {p}", g, o, A=A, T=c["T"],
                      n_valid=c["n_valid"], mode=modes[c["mode"]], row_dtype=row_dtype,
                      bf16_stats=bf, rlp=float(c["rlp"][p]))
            checked += 1
    assert checked >= 60, checked
    bf16_bar(bf, "emulated random rows")


def read_lmhead(path):
    b = open(path, "rb").read()
    o = 0

    def take(dt, n):
        nonlocal o
        a = np.frombuffer(b, dt, n, o)
        o += a.nbytes
        return a
    n, V, d, K, chunk, dzs = (int(v) for v in take(np.int32, 6))
    r = dict(n=n, V=V, d=d, K=K, chunk=chunk)
    bf = lambda u: (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # noqa: E731
    r["x"] = bf(take(np.uint16, n * d)).reshape(n, d)
    r["w"] = bf(take(np.uint16, V * d)).reshape(V, d)
    r["ids"] = take(np.int32, n * K).reshape(n, K)
    r["q"] = take(np.float32, n * K).reshape(n, K)
    r["sampled"] = take(np.int32, n)
    r["resp"] = take(np.int32, n)
    r["adv"] = take(np.float32, 4)
    r["n_valid"] = int(take(np.int64, 1)[0])
    r["z"] = take(np.float32, n * V).reshape(n, V)
    r["stats"] = take(np.float32, n * 16).reshape(n, 16)
    r["idx"] = take(np.int32, n * 2).reshape(n, 2)
    r["hl"] = take(np.float32, n * K).reshape(n, K)
    r["dz"] = take(np.uint16, n * dzs).reshape(n, dzs)[:, :V]
    r["dh"] = take(np.float32, n * d).reshape(n, d)
    r["dw"] = take(np.float32, V * d).reshape(V, d)
    r["status"] = int(take(np.uint32, 1)[0])
    return r


def test_lmhead_entry_points_match_oracle_under_sanitizers(harness, tmp_path):
    path = tmp_path / "lmhead.bin"
    # 260 rows (two row tiles), 300 ids (two vocabulary tiles, ragged),
    # d = 64, K = 8, backward chunks of 100 rows (three, the last ragged)
    run(harness, "lmhead", path, 260, 300, 64, 8, 100)
    r = read_lmhead(path)
    assert r["status"] == 0
    x, w, d = r["x"], r["w"], r["d"]
    # the GEMM's logits against the float64 product
    err = np.abs(r["z"] - O.lmhead_logits(x, w))
    bound = (d + 16) * 2.0 ** -24 * (np.abs(x) @ np.abs(w).T)
    assert np.all(err <= bound), float(err.max())
    # statistics on the emulated logits, at the row kernels' tolerances;
    # the sc_center columns need q and the advantages: checked through the
    # dLogits rows below
    G = np.zeros((r["n"], r["V"]))
    for p in range(r["n"]):
        if r["resp"][p] < 0:
            assert list(r["idx"][p]) == [-1, -1]
            continue
        o = O.sc_row(r["z"][p].astype(np.float64), 1.0, r["ids"][p], r["q"][p],
                     int(r["sampled"][p]))
        check_row(f"emulated lmhead row {p}",
                  dict(stats=r["stats"][p], idx=r["idx"][p], head_logp=r["hl"][p]), o,
                  stats_only=True)
        G[p] = O.sc_row(r["z"][p].astype(np.float64), 1.0, r["ids"][p], r["q"][p],
                        int(r["sampled"][p]), advantage=float(r["adv"][r["resp"][p]]),
                        n_valid=r["n_valid"], row_mode=O.MODE_DLOGITS)["row"]
    dist, eq = compare_bf16(r["dz"], G)
    assert dist <= 1 and eq >= MIN_BF16_EQUAL, (dist, eq)
    # gradients: the GPU tests' bound (bf16 rounding of dZ plus fp32 sums)
    rdX, rdW = O.lmhead_backward(x, w, G)
    tol_x = 2.0 ** -8 * (np.abs(G) @ np.abs(w)) + 1e-30
    tol_w = 2.0 ** -8 * (np.abs(G).T @ np.abs(x)) + 1e-30
    assert np.all(np.abs(r["dh"] - rdX) <= tol_x), float(np.abs(r["dh"] - rdX).max())
    assert np.all(np.abs(r["dw"] - rdW) <= tol_w), float(np.abs(r["dw"] - rdW).max())


def read_record(path):
    b = open(path, "rb").read()
    o = 0

    def take(dt, n):
        nonlocal o
        a = np.frombuffer(b, dt, n, o)
        o += a.nbytes
        return a
    cases = []
    while o < len(b):
        n, V, K, stride, dtype, with_sampled = (int(v) for v in take(np.int32, 6))
        c = dict(n=n, V=V, K=K, with_sampled=bool(with_sampled), T=float(take(np.float32, 1)[0]))
        z = take(np.float32, n * stride).reshape(n, stride)[:, :V]
        if dtype == SC_BF16:
            z = torch.from_numpy(z.copy()).to(torch.bfloat16).float().numpy()
        c["z"] = z.astype(np.float64)
        c["sampled"] = take(np.int32, n)
        c["ids"] = take(np.int32, n * K).reshape(n, K)
        c["probs"] = take(np.float32, n * K).reshape(n, K)
        c["lp"] = take(np.float32, n)
        cases.append(c)
    return cases


def test_record_matches_oracle_under_sanitizers(harness, tmp_path):
    """sc_record on 24 seeded random cases in the emulated device
    environment, every row against the oracle: ids exact, probabilities
    within abs 1e-6 + rel 4e-6, the sampled log-probability within abs
    1e-5 (or one fp32 spacing of it)."""
    path = tmp_path / "record.bin"
    out = run(harness, "record", path, 24, 5)
    assert out.count("record case") == 24
    cases = read_record(path)
    assert len(cases) == 24
    rows = flagged = big_k = 0
    for ci, c in enumerate(cases):
        for r in range(c["n"]):
            a = int(c["sampled"][r]) if c["with_sampled"] else None
            o = O.record_topk(c["z"][r], c["T"], c["K"], sampled=a)
            tag = f"emulated record case {ci} row {r}"
            if o["flags"]:
                assert np.all(c["ids"][r] == -1) and np.all(np.isnan(c["probs"][r])), tag
                flagged += 1
                continue
            np.testing.assert_array_equal(c["ids"][r], o["head_ids"], err_msg=tag)
            err = np.abs(c["probs"][r] - o["head_probs"]) - (1e-6 + 4e-6 * o["head_probs"])
            assert err.max() <= 0, (tag, float(np.abs(c["probs"][r] - o["head_probs"]).max()))
            if a is not None:
                tol = max(1e-5, float(np.spacing(np.float32(abs(o["sampled_logp"])))))
                assert abs(c["lp"][r] - o["sampled_logp"]) <= tol, (tag, c["lp"][r],
                                                                    o["sampled_logp"])
            rows += 1
            big_k += c["K"] > 256
    print(f"[case] emulated record: {rows} rows checked, {flagged} flagged, "
          f"{big_k} with K > 256", flush=True)
    assert rows >= 30 and big_k >= 3, (rows, big_k)
