#!/usr/bin/env python3
"""Throughput of the score-centering (SC) correction on one MI355X.

One step is the whole per-position path over the quick-check workload
(2 prompts x 4 responses x 1,024 tokens = 8,192 positions, V = 248,320,
K = 128, bf16 trainer logits): exact valid-token count, group
normalisation of the rewards, the fused correction kernel (trainer softmax
statistics, gathers, mu_hat, loss, diagnostics and the bf16 dLogits row of
every position) and the step reductions.  Inputs are resident in HBM before
the timed region starts.

Prints one JSON line.  Besides the throughput it reports the dominant
kernel's roofline position (algorithmic bytes / its own event-timed launch
duration) and the CPU oracle's throughput on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import multiprocessing as mp
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SC positions/sec at V=248,320 K=128 (1 GPU); achieved HBM GB/s vs peak"
VOCAB, K = 248_320, 128
PROMPTS, GROUP, TOKENS = 2, 4, 1024
N_ROWS = PROMPTS * GROUP * TOKENS
HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X published dense bf16 matrix peak
LM_ROWS, LM_D = 16_384, 4096    # fused LM-head slice (64 x 8,800-token batch, d = 4,096)
PROFILE = os.path.join(ROOT, "profiles", "sc_correct_quick_check_pmc.md")
# Everything that shapes the fused row kernel whose counters profiles/ holds:
# its sources, the header with its launch-shape macros, and the build flags.
KERNEL_SOURCES = [os.path.join(ROOT, "off_policy_logit_amd", "csrc", f)
                  for f in ("sc_kernels.hip", "sc_device.h", "sc_internal.h")]

# Algorithmic bytes of one position through the fused kernel (sc_correct with
# a bf16 dLogits row): logits 2V, head ids 4K, head probs 4K, sampled,
# resp_idx, rollout logp, advantage (4 B each) read; dLogits 2V, head logp 4K,
# coefficients 4K, 16 fp32 statistics and 2 int32 indices written.
BYTES_PER_POSITION = 2 * VOCAB + 8 * K + 16 + 2 * VOCAB + 8 * K + 64 + 8
# Stats-only pass (sc_logprobs): logits 2V, ids 4K, sampled, resp_idx read;
# log p at H 4K, 5 of the statistics and 2 indices written.
BYTES_PER_POSITION_STATS = 2 * VOCAB + 4 * K + 8 + 4 * K + 20 + 8
# Rollout-side record (sc_record): logits 2V and the sampled id read; ids 4K,
# probabilities 4K and the sampled log-probability written.
BYTES_PER_POSITION_RECORD = 2 * VOCAB + 4 + 8 * K + 4


def source_digest():
    from off_policy_logit_amd import build as B
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    # include paths relative to the repository: the same tree can sit at
    # another absolute path (where the bench runs)
    flags = [os.path.relpath(f, ROOT) if os.path.isabs(f) else f for f in B.FLAGS]
    h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per launch from the committed PMC summary, or None when the
    kernel sources changed since the counters were taken."""
    if not os.path.exists(PROFILE):
        return None
    text = open(PROFILE).read()
    m_bytes = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    m_src = re.search(r"kernel_source_digest:\s*([0-9a-f]+)", text)
    if not (m_bytes and m_src) or m_src.group(1) != source_digest():
        return None
    return float(m_bytes.group(1))


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------
_SAMPLE = None


def _oracle_rows(idx):
    from oracle import sc_oracle as O
    z, ids, q, a, rlp = _SAMPLE
    for i in idx:
        O.sc_row(z[i], 1.0, ids[i], q[i], a[i], rollout_logp=rlp[i],
                 advantage=0.5, n_valid=N_ROWS, row_mode=O.MODE_DLOGITS)
    return len(idx)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(rows, min_seconds=10.0, max_passes=200, single_seconds=4.0):
    """Time the oracle on `rows` positions generated on the host with the
    quick-check generator: first on one thread in this process for about
    `single_seconds`, then in passes over the sample until `min_seconds` of
    wall time have elapsed in a fork pool of one process per available core
    (capped at 16).  Runs before anything touches the GPU."""
    global _SAMPLE
    import synthetic
    spec = synthetic.BigSpec(seed=1)
    parts = [synthetic.big_chunk(spec, min(128, rows - r0), 9000 + r0, "cpu")
             for r0 in range(0, rows, 128)]
    z = np.concatenate([p["logits"].float().numpy() for p in parts])
    ids = np.concatenate([p["head_ids"].numpy() for p in parts])
    q = np.concatenate([p["head_probs"].numpy() for p in parts])
    a = np.concatenate([p["sampled"].numpy() for p in parts])
    rlp = np.concatenate([p["rollout_logp"].numpy() for p in parts])
    _SAMPLE = (z, ids, q, a, rlp)
    one, t1 = 0, time.perf_counter()
    while time.perf_counter() - t1 < single_seconds and one < rows:
        one += _oracle_rows([one])
    single = one / (time.perf_counter() - t1)
    cores = min(16, len(os.sched_getaffinity(0)))
    chunks = [list(range(i, rows, cores)) for i in range(cores)]
    ctx = mp.get_context("fork")
    done, passes = 0, 0
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        while passes < max_passes:
            done += sum(pool.map(_oracle_rows, chunks))
            passes += 1
            if time.perf_counter() - t0 >= min_seconds:
                break
    dt = time.perf_counter() - t0
    _SAMPLE = None
    return dict(value=round(done / dt, 1), unit="positions/s", cores=cores, kind="oracle",
                cpu_model=cpu_model(), single_thread_value=round(single, 1),
                sample=f"{rows} positions of the quick-check workload (V={VOCAB}, K={K}, "
                       f"bf16 logits) x {passes} passes = {done} positions, full "
                       f"per-position outputs incl. the dLogits row, float64, "
                       f"{dt:.1f} s wall on {cores} processes; single thread: {one} "
                       f"positions in this process")


# ---------------------------------------------------------------------------
# GPU
# ---------------------------------------------------------------------------
def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def full_step_measure(dev, reps, chunks=32, chunk_rows=16_384):
    """The full-step workload: 32 prompts x 4 responses x 4,096 tokens =
    524,288 positions, response lengths uniform in [256, 4,096] and the rest
    padding, in 32 chunks of 16,384 positions.  The exact valid count runs
    once over the step's response indices; then each chunk is generated into
    HBM (untimed) and its fused kernel (bf16 dLogits) and step sums are timed
    `reps` times.  The step time is the count plus the sum of the chunk
    times."""
    import torch
    import synthetic
    from off_policy_logit_amd import sc
    lengths = synthetic.full_step_lengths()
    rows_all = torch.arange(chunks * chunk_rows)
    lens = torch.as_tensor(np.asarray(lengths))[rows_all // 4096]
    resp_all = torch.where(rows_all % 4096 < lens, rows_all // 4096, -1).to(torch.int32).to(dev)
    n_valid = torch.empty(1, dtype=torch.int64, device=dev)
    sc.count_valid(resp_all, out=n_valid)
    torch.cuda.synchronize()
    e0, e1 = _events()
    e0.record()
    for _ in range(reps):
        sc.count_valid(resp_all, out=n_valid)
    e1.record()
    torch.cuda.synchronize()
    count_ms = e0.elapsed_time(e1) / reps
    valid = int(n_valid.item())
    g = torch.Generator().manual_seed(12)
    adv = torch.randn(int(resp_all.max().item()) + 1, generator=g).to(dev)
    batch = torch.empty(sc.NBATCH, dtype=torch.float64, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    dz = torch.empty(chunk_rows, VOCAB, dtype=torch.bfloat16, device=dev)
    out = None
    chunk_ms, byte_total = [], 0
    for ck in range(chunks):
        c = synthetic.full_step_chunk(dev, ck, lengths, chunk_rows=chunk_rows)
        resp = resp_all[ck * chunk_rows:(ck + 1) * chunk_rows]
        assert torch.equal(resp, c["resp_idx"])
        kw = dict(n_valid=n_valid, rollout_logp=c["rollout_logp"], row_out=dz,
                  dev_status=status)
        if out is None:
            out = sc.correct(c["logits"], c["head_ids"], c["head_probs"], c["sampled"], resp,
                             adv, **kw)
        sc.correct(c["logits"], c["head_ids"], c["head_probs"], c["sampled"], resp, adv,
                   out=out, coef=out["coef"], **kw)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            sc.correct(c["logits"], c["head_ids"], c["head_probs"], c["sampled"], resp, adv,
                       out=out, coef=out["coef"], **kw)
            sc.batch_sums(out["row_stats"], resp, n_valid, out=batch, accumulate=ck > 0)
        e1.record()
        torch.cuda.synchronize()
        chunk_ms.append(e0.elapsed_time(e1) / reps)
        nv = int((resp >= 0).sum().item())
        # valid rows move the fused kernel's bytes; padding rows only write a zero row
        byte_total += nv * BYTES_PER_POSITION + (chunk_rows - nv) * (2 * VOCAB + 8 * K + 72)
        del c
    if int(status.item()) != 0:
        raise RuntimeError(f"full-step device status {int(status.item())}")
    del dz, out
    torch.cuda.empty_cache()
    total_ms = count_ms + sum(chunk_ms)
    return {"workload": f"full step: {chunks} chunks x {chunk_rows} = {chunks * chunk_rows} "
                        f"positions, {valid} valid, V={VOCAB}, K={K}, bf16 logits and dLogits",
            "step_ms": round(total_ms, 3), "count_ms": round(count_ms, 4),
            "chunk_ms_min": round(min(chunk_ms), 4), "chunk_ms_max": round(max(chunk_ms), 4),
            "valid_positions_per_s": round(valid / (total_ms * 1e-3), 1),
            "GBps": round(byte_total / (sum(chunk_ms) * 1e-3) / 1e9, 1)}


def stress_measure(dev, reps, chunks=8, chunk_rows=16_384):
    """Distribution stress: 131,072 positions (8 chunks of 16,384: thirds
    peaked x8, flat x0.1 and mixed; 5% of sampled tokens outside the head)
    per rollout-noise sigma in {0.01, 0.1, 0.5}; each chunk generated into
    HBM (untimed), then the fused kernel with bf16 dLogits timed `reps`
    times."""
    import torch
    import synthetic
    from off_policy_logit_amd import sc
    res = {}
    adv = torch.tensor([0.5], device=dev)
    n_valid = torch.tensor([chunks * chunk_rows], dtype=torch.int64, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    dz = torch.empty(chunk_rows, VOCAB, dtype=torch.bfloat16, device=dev)
    e0, e1 = _events()
    for sigma in (0.01, 0.1, 0.5):
        ms, out = [], None
        for ck in range(chunks):
            c = synthetic.stress_chunk(dev, ck, sigma, chunk_rows=chunk_rows)
            kw = dict(n_valid=n_valid, rollout_logp=c["rollout_logp"], row_out=dz,
                      dev_status=status)
            args = (c["logits"], c["head_ids"], c["head_probs"], c["sampled"], c["resp_idx"],
                    adv)
            out = sc.correct(*args, out=out, coef=None if out is None else out["coef"], **kw)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                sc.correct(*args, out=out, coef=out["coef"], **kw)
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1) / reps)
            del c
        if int(status.item()) != 0:
            raise RuntimeError(f"stress device status {int(status.item())}")
        tot = sum(ms)
        res[f"sigma={sigma}"] = {"kernel_ms_total": round(tot, 3),
                                 "positions_per_s": round(chunks * chunk_rows / (tot * 1e-3), 1),
                                 "GBps": round(chunks * chunk_rows * BYTES_PER_POSITION /
                                               (tot * 1e-3) / 1e9, 1)}
    del dz
    torch.cuda.empty_cache()
    return {"workload": f"distribution stress: {chunks * chunk_rows} positions per sigma, "
                        f"V={VOCAB}, K={K}, bf16 logits and dLogits", **res}


def lmhead_measure(dev, reps):
    """Fused LM-head statistics (sc_logprobs_lmhead) on a 16,384-row slice at
    V = 248,320, d = 4,096: event-timed average of the three kernels, in
    positions/s and dense bf16 TFLOP/s (2 d V per position)."""
    import torch
    import synthetic
    from off_policy_logit_amd import sc
    w, wr = synthetic.lmhead_weights(dev, vocab=VOCAB, d=LM_D, seed=5)
    c = synthetic.lmhead_chunk(dev, wr, LM_ROWS, seed=6)
    del wr
    ws = torch.empty(sc.lmhead_workspace_size(LM_ROWS, VOCAB, K), dtype=torch.uint8, device=dev)
    out = dict(row_stats=torch.empty(LM_ROWS, sc.NSTATS, device=dev),
               row_idx=torch.empty(LM_ROWS, 2, dtype=torch.int32, device=dev),
               head_logp=torch.empty(LM_ROWS, K, device=dev))
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def run():
        sc.logprobs_lmhead(c["hidden"], w, c["head_ids"], c["sampled"], None, out=out,
                           workspace=ws, dev_status=status)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError(f"lmhead device status {int(status.item())}")
    ms = e0.elapsed_time(e1) / reps
    tflops = 2.0 * LM_D * VOCAB * LM_ROWS / (ms * 1e-3) / 1e12

    # backward through the head: dLogits recomputed chunk by chunk (8,192
    # rows), dHidden = dZ W and dW = dZ^T X; 3 x 2 d V flop per position
    resp = torch.zeros(LM_ROWS, dtype=torch.int32, device=dev)
    adv = torch.ones(1, device=dev)
    n_valid = torch.tensor([LM_ROWS], dtype=torch.int64, device=dev)
    sc.center(out, c["head_ids"], c["head_probs"], c["sampled"], resp, adv,
              n_valid=n_valid, rollout_logp=c["rollout_logp"], vocab=VOCAB)
    dh = torch.empty(LM_ROWS, LM_D, dtype=torch.bfloat16, device=dev)
    dW = torch.empty(VOCAB, LM_D, device=dev)
    bws = torch.empty(sc.lib().sc_lmhead_backward_workspace_size(8192, VOCAB, LM_D),
                      dtype=torch.uint8, device=dev)

    def back():
        sc.lmhead_backward(c["hidden"], w, out, c["head_ids"], c["head_probs"], c["sampled"],
                           resp, adv, n_valid, d_hidden=dh, d_weight=dW, chunk_rows=8192,
                           workspace=bws)
    back()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        back()
    e1.record()
    torch.cuda.synchronize()
    bms = e0.elapsed_time(e1) / reps
    btflops = 3 * 2.0 * LM_D * VOCAB * LM_ROWS / (bms * 1e-3) / 1e12
    del w, c, ws, dh, dW, bws
    torch.cuda.empty_cache()
    return {"workload": f"{LM_ROWS} rows x V={VOCAB} x d={LM_D}, bf16 hidden and "
                        "projection, K=128, logits never stored",
            "kernel_ms": round(ms, 3), "positions_per_s": round(LM_ROWS / (ms * 1e-3), 1),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)},
            "backward": {"ms": round(bms, 3),
                         "positions_per_s": round(LM_ROWS / (bms * 1e-3), 1),
                         "note": "dLogits recompute + dHidden and dW products, all on "
                                 "this library's MFMA loop, 8,192-row chunks",
                         "roofline": {"bound": "mfma", "achieved": round(btflops, 1),
                                      "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                      "frac": round(btflops / MFMA_BF16_PEAK_TFLOPS, 4)}}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-rows", type=int, default=512,
                    help="positions in the CPU-oracle sample (0 skips it)")
    ap.add_argument("--no-lmhead", action="store_true",
                    help="skip the fused LM-head measurement")
    ap.add_argument("--no-full-step", action="store_true",
                    help="skip the full-step workload (32 chunks)")
    ap.add_argument("--no-stress", action="store_true",
                    help="skip the distribution-stress workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device copy before the timed region "
                         "(reference kernel for PMC byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    cpu = cpu_baseline(args.cpu_rows) if args.cpu_rows > 0 else None

    import torch
    import synthetic
    from off_policy_logit_amd import sc

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = synthetic.quick_check(dev, n_prompts=PROMPTS, group_size=GROUP, tokens=TOKENS)
    n = d["logits"].shape[0]
    assert n == N_ROWS and d["logits"].shape[1] == VOCAB
    dlogits = torch.empty(n, VOCAB, dtype=torch.bfloat16, device=dev)
    out = dict(row_stats=torch.empty(n, sc.NSTATS, device=dev),
               row_idx=torch.empty(n, 2, dtype=torch.int32, device=dev),
               head_logp=torch.empty(n, K, device=dev))
    coef = torch.empty(n, K, device=dev)
    n_valid = torch.empty(1, dtype=torch.int64, device=dev)
    adv = torch.empty_like(d["rewards"])
    batch = torch.empty(sc.NBATCH, dtype=torch.float64, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ev = []

    def step(timed):
        sc.count_valid(d["resp_idx"], out=n_valid)
        sc.group_norm(d["rewards"], GROUP, out=adv)
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        sc.correct(d["logits"], d["head_ids"], d["head_probs"], d["sampled"],
                   d["resp_idx"], adv, n_valid=n_valid, rollout_logp=d["rollout_logp"],
                   row_out=dlogits, row_mode=sc.ROW_DLOGITS, out=out, coef=coef,
                   dev_status=status)
        if timed:
            e1.record()
            ev.append((e0, e1))
        sc.batch_sums(out["row_stats"], d["resp_idx"], n_valid, out=batch)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    if int(status.item()) != 0:
        raise RuntimeError(f"device status {int(status.item())}")
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))

    # stats-only pass (sc_logprobs), secondary line
    st = dict(row_stats=out["row_stats"], row_idx=out["row_idx"], head_logp=out["head_logp"])
    for _ in range(3):
        sc.logprobs(d["logits"], d["head_ids"], d["sampled"], d["resp_idx"], out=st)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(5, args.steps // 2)
    e0.record()
    for _ in range(reps):
        sc.logprobs(d["logits"], d["head_ids"], d["sampled"], d["resp_idx"], out=st)
    e1.record()
    torch.cuda.synchronize()
    stats_ms = e0.elapsed_time(e1) / reps

    # reference rate of the memory system for the same traffic shape: a plain
    # device copy of the logits into the dLogits buffer (reads and writes the
    # fused kernel's algorithmic bytes, with no arithmetic)
    dlogits.copy_(d["logits"])
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dlogits.copy_(d["logits"])
    e1.record()
    torch.cuda.synchronize()
    copy_ms = e0.elapsed_time(e1) / reps
    copy_bytes = 2 * d["logits"].numel() * d["logits"].element_size()
    # the library's reference copy kernel on the same bytes (nontemporal
    # 16-byte stream, one workgroup per 512 KiB): the measured copy ceiling
    sc.reference_copy(d["logits"], dlogits)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        sc.reference_copy(d["logits"], dlogits)
    e1.record()
    torch.cuda.synchronize()
    ref_copy_ms = e0.elapsed_time(e1) / reps
    ref_copy_gbps = copy_bytes / (ref_copy_ms * 1e-3) / 1e9

    # two-call path: sc_logprobs, then sc_center streaming the logits again
    # for the dLogits row (the same outputs as the fused kernel)
    def two_call():
        sc.logprobs(d["logits"], d["head_ids"], d["sampled"], d["resp_idx"], out=st)
        sc.center(st, d["head_ids"], d["head_probs"], d["sampled"], d["resp_idx"], adv,
                  n_valid=n_valid, rollout_logp=d["rollout_logp"], logits=d["logits"],
                  row_out=dlogits, row_mode=sc.ROW_DLOGITS, coef=coef, dev_status=status)
    for _ in range(2):
        two_call()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        two_call()
    e1.record()
    torch.cuda.synchronize()
    two_ms = e0.elapsed_time(e1) / reps
    if int(status.item()) != 0:
        raise RuntimeError(f"two-call device status {int(status.item())}")

    # rollout-side record (sc_record) on the same logits, secondary line
    rec = dict(head_ids=torch.empty(n, K, dtype=torch.int32, device=dev),
               head_probs=torch.empty(n, K, device=dev),
               sampled_logp=torch.empty(n, device=dev))
    for _ in range(2):
        sc.record(d["logits"], K, sampled=d["sampled"], dev_status=status, **rec)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        sc.record(d["logits"], K, sampled=d["sampled"], dev_status=status, **rec)
    e1.record()
    torch.cuda.synchronize()
    rec_ms = e0.elapsed_time(e1) / reps
    if int(status.item()) != 0:
        raise RuntimeError(f"record device status {int(status.item())}")

    del d, dlogits, out, coef, st, rec
    torch.cuda.empty_cache()
    full = None if args.no_full_step else full_step_measure(dev, 3)
    stress = None if args.no_stress else stress_measure(dev, 3)
    lm = None if args.no_lmhead else lmhead_measure(dev, max(3, args.steps // 10))

    bytes_launch = n * BYTES_PER_POSITION
    achieved = bytes_launch / (kern_ms * 1e-3) / 1e9
    traffic = traffic_from_profile()
    value = args.steps * n / dt
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "quick-check: 2 prompts x 4 responses x 1024 tokens "
                               "= 8192 positions, V=248320, K=128, bf16 logits in, "
                               "bf16 dLogits out",
                   "positions": n, "vocab": VOCAB, "k": K,
                   "logits_dtype": "bf16", "dlogits_dtype": "bf16"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "copy_reference_GBps": round(ref_copy_gbps, 1),
                     "frac_of_copy": round(achieved / ref_copy_gbps, 4),
                     "kernel": "sc_correct (k_row bf16->bf16, fused)",
                     "kernel_ms": round(kern_ms, 4),
                     "bytes_per_launch": bytes_launch},
        "cpu_baseline": cpu,
        "secondary": {
            "stats_only_positions_per_s": round(n / (stats_ms * 1e-3), 1),
            "stats_only_kernel_ms": round(stats_ms, 4),
            "stats_only_GBps": round(n * BYTES_PER_POSITION_STATS / (stats_ms * 1e-3) / 1e9, 1),
            "copy_same_bytes_ms": round(copy_ms, 4),
            "copy_GBps": round(copy_bytes / (copy_ms * 1e-3) / 1e9, 1),
            "reference_copy_ms": round(ref_copy_ms, 4),
            "stats_only_frac_of_copy": round(n * BYTES_PER_POSITION_STATS / (stats_ms * 1e-3) /
                                             1e9 / ref_copy_gbps, 4),
            "two_call_positions_per_s": round(n / (two_ms * 1e-3), 1),
            "two_call_ms": round(two_ms, 4),
            "record_positions_per_s": round(n / (rec_ms * 1e-3), 1),
            "record_kernel_ms": round(rec_ms, 4),
            "record_GBps": round(n * BYTES_PER_POSITION_RECORD / (rec_ms * 1e-3) / 1e9, 1),
            "full_step": full,
            "stress": stress,
            "lmhead": lm,
        },
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
