"""sc_logprobs_lmhead_static, the LM-head statistics entry point that
allocates nothing, against sc_logprobs_lmhead on the same inputs.

Both run the same kernels; the static one takes its workspace from the
library's per-GPU static array, which keeps the previous call's contents.
Two calls in a row at the full vocabulary (248,320 x 4096), the first at the
largest row count the array holds and the second smaller and ragged, must
give bit-identical outputs; a request one row beyond the limit is refused on
the host and leaves the outputs untouched.
"""
import pytest
import torch

import synthetic

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from off_policy_logit_amd import sc

DEV = "cuda:0"
V, D, K = 248_320, 4096, 128
MAX_ROWS = 11_881          # largest row count whose workspace fits the array


def say(*a):
    print("[case]", *a, flush=True)


def bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def same(a, b):
    return torch.equal(bits(a), bits(b))


@pytest.fixture(scope="module")
def weights():
    w, wr = synthetic.lmhead_weights(DEV, vocab=V, d=D, seed=31)
    yield w, wr
    del w, wr
    torch.cuda.empty_cache()


def run_both(w, c, resp, T):
    n = c["hidden"].shape[0]
    assert sc.lmhead_workspace_size(n, V, K) <= sc.STATIC_SCRATCH_BYTES
    st_a = torch.zeros(1, dtype=torch.int32, device=DEV)
    st_b = torch.zeros(1, dtype=torch.int32, device=DEV)
    # Same sentinel in both: columns the entry point does not write compare equal.
    a, b = (dict(row_stats=torch.full((n, sc.NSTATS), -7.0, device=DEV),
                 row_idx=torch.full((n, 2), -9, dtype=torch.int32, device=DEV),
                 head_logp=torch.full((n, K), -7.0, device=DEV)) for _ in range(2))
    sc.logprobs_lmhead_static(c["hidden"], w, c["head_ids"], c["sampled"], resp,
                              temperature=T, out=a, dev_status=st_a)
    sc.logprobs_lmhead(c["hidden"], w, c["head_ids"], c["sampled"], resp,
                       temperature=T, out=b, dev_status=st_b)
    torch.cuda.synchronize()
    for key in ("row_stats", "row_idx", "head_logp"):
        assert same(a[key], b[key]), key
    assert same(st_a, st_b)
    return a


def test_static_matches_workspace_entry_point_on_two_calls(weights):
    w, wr = weights
    # First call: the largest request the static array holds.
    say(f"static lmhead call 1: rows={MAX_ROWS} V={V} d={D} k={K}")
    c = synthetic.lmhead_chunk(DEV, wr, MAX_ROWS, seed=32)
    resp = torch.zeros(MAX_ROWS, dtype=torch.int32, device=DEV)
    resp[7] = -1
    resp[5000:5040] = -1
    c["head_ids"][9, 4] = c["head_ids"][9, 2]           # duplicate id
    c["sampled"][11] = V                                # sampled id out of range
    out = run_both(w, c, resp, 1.0)
    st, ix = out["row_stats"].cpu(), out["row_idx"].cpu()
    assert float(st[7, 0]) == 0.0 and ix[7].tolist() == [-1, -1]       # padding row
    assert bool(torch.isnan(st[9, 0])) and bool(torch.isnan(st[11, 0]))  # flagged rows
    assert bool(torch.isfinite(st[12, [0, 1, 2, 3, 11]]).all()) and ix[12, 0] >= 0
    del c, resp, out
    # Second call: smaller and ragged, at another temperature, on the array
    # the first call left behind.
    n2 = 777
    say(f"static lmhead call 2: rows={n2} T=0.7")
    c = synthetic.lmhead_chunk(DEV, wr, n2, seed=33, temperature=0.7)
    run_both(w, c, None, 0.7)

    # One row beyond the limit: refused before any launch, outputs untouched.
    n3 = MAX_ROWS + 1
    say(f"static lmhead refused: rows={n3}")
    x = torch.zeros(n3, D, dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros(n3, K, dtype=torch.int32, device=DEV)
    ids[:] = torch.arange(K, dtype=torch.int32, device=DEV)
    samp = torch.zeros(n3, dtype=torch.int32, device=DEV)
    o = dict(row_stats=torch.full((n3, sc.NSTATS), 3.0, device=DEV),
             row_idx=torch.full((n3, 2), 5, dtype=torch.int32, device=DEV))
    with pytest.raises(sc.ScError, match="SC_ERR_TOO_LARGE"):
        sc.logprobs_lmhead_static(x, w, ids, samp, out=o)
    torch.cuda.synchronize()
    assert bool((o["row_stats"] == 3.0).all()) and bool((o["row_idx"] == 5).all())
