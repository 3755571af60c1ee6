"""HIP graph capture of one training-step pass of the SC path.

The library allocates nothing and issues no memset, so its launches can be
captured into a HIP graph.  The graph (count, group norm, the fused
correction with bf16 dLogits, step sums) is replayed several times with
eager work and synchronisations in between; every replay must reproduce
the eager run bit for bit (the kernels are deterministic).
"""
import numpy as np
import pytest
import torch

import synthetic

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from off_policy_logit_amd import sc

DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)


def test_step_graph_replays_match_eager():
    say("graph capture of count/group-norm/correct/batch-sums on the tiny workload (bf16)")
    h = synthetic.tiny(seed=3)
    d = {k: (torch.from_numpy(np.ascontiguousarray(v)).to(DEV) if isinstance(v, np.ndarray) else v)
         for k, v in h.items()}
    logits = d["logits"].to(torch.bfloat16)
    n, V = logits.shape
    k = d["head_ids"].shape[1]
    n_valid = torch.empty(1, dtype=torch.int64, device=DEV)
    adv = torch.empty_like(d["rewards"])
    out = dict(row_stats=torch.empty(n, sc.NSTATS, device=DEV),
               row_idx=torch.empty(n, 2, dtype=torch.int32, device=DEV),
               head_logp=torch.empty(n, k, device=DEV))
    coef = torch.empty(n, k, device=DEV)
    row = torch.empty(n, V, dtype=torch.bfloat16, device=DEV)
    batch = torch.empty(sc.NBATCH, dtype=torch.float64, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)

    def step():
        sc.count_valid(d["resp_idx"], out=n_valid)
        sc.group_norm(d["rewards"], h["group_size"], out=adv)
        sc.correct(logits, d["head_ids"], d["head_probs"], d["sampled"], d["resp_idx"], adv,
                   n_valid=n_valid, rollout_logp=d["rollout_logp"], row_out=row, out=out,
                   coef=coef, dev_status=status)
        sc.batch_sums(out["row_stats"], d["resp_idx"], n_valid, out=batch)

    step()
    torch.cuda.synchronize()
    ref = {key: v.clone() for key, v in out.items()}
    ref_row, ref_batch, ref_coef = row.clone(), batch.clone(), coef.clone()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                       # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        say(f"graph replay {rep}")
        for v in list(out.values()) + [row, batch, coef]:
            v.fill_(7)               # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        for key in ref:
            assert torch.equal(out[key].view(torch.int32), ref[key].view(torch.int32)), key
        assert torch.equal(row.view(torch.int16), ref_row.view(torch.int16))
        assert torch.equal(coef.view(torch.int32), ref_coef.view(torch.int32))
        assert torch.equal(batch.view(torch.int64), ref_batch.view(torch.int64))
