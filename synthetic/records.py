"""Seeded synthetic inputs for the score-centering (SC) path.

This module emulates the *producer* of the SC inputs: a rollout engine that
samples a token from its own (slightly different, low-precision) distribution
and records the top-K candidate ids with their probabilities plus the sampled
token's log-probability (Score Centering page, section "Score Centering").  It
also draws trainer logits, rewards and response lengths.  It never computes
anything on the trainer side of the method, and both the HIP path and the CPU
oracle read its outputs; it imports neither of them.

Shapes and distributions follow the workloads of the pages: groups of 4
responses per prompt (2 x 4 for the quick check, 32 x 4 for the full step;
Agent Lightning release note, section 2, and the Score Centering page,
section "Training"), K = 128 recorded candidates, temperature 1, bf16 trainer
logits, and the 64 x 8,800-token repair-run batch of the lecture notes
("RL systems for agents", section 0).  The vocabulary size 248,320 is a
workload parameter.

Workloads (every draw is seeded):

* ``tiny``: 8 groups x 4 responses x 8 tokens = 256 positions, V = 4,096,
  fp32 logits ~ N(0, 2^2); rollout logits = trainer + N(0, 0.05^2).
* ``big_chunk`` (quick-check / full-step / stress generators): bf16 logits
  z = bf16(scale * (N(0, sd^2) + b_v)) with a Zipf(1.1) per-id bias
  b_v = -1.1 ln(rank_v) over a seeded permutation of ranks; rollout logits
  zr = z + N(0, noise^2) in fp32.
* ``lmhead_weights`` / ``lmhead_chunk`` (fused LM-head workload, 64 x 8,800
  positions in the lecture notes' repair batch, d = 4,096): hidden states
  bf16(N(0, 1)), vocabulary projection bf16(N(0, 0.02^2)) (logit std about
  1.28), the rollout scoring with bf16(W + N(0, 1e-3^2)).
* In all of them H = top-K ids of the rollout softmax at temperature T,
  q = the rollout probabilities there (fp32), the sampled token is drawn from
  the rollout softmax by the Gumbel-max rule, and its rollout log-probability
  is recorded in fp32.  Rewards are Bernoulli(0.5) per response.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

VOCAB = 248_320
TOPK = 128


# --------------------------------------------------------------------------
# Tiny workload (host numpy)
# --------------------------------------------------------------------------
def tiny(seed=0, temperature=1.0, n_groups=8, group_size=4, tokens=8,
         vocab=4096, k=TOPK):
    """The 256-position tiny workload as numpy arrays (fp32 logits)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n_resp = n_groups * group_size
    n = n_resp * tokens
    z = rng.normal(0.0, 2.0, size=(n, vocab)).astype(np.float32)
    zr = z.astype(np.float64) + rng.normal(0.0, 0.05, size=(n, vocab))
    ur = zr / float(temperature)
    mx = ur.max(axis=1, keepdims=True)
    lr = ur - (mx + np.log(np.exp(ur - mx).sum(axis=1, keepdims=True)))
    # top-K by probability, ties to the lower id (stable sort of -log prob)
    order = np.argsort(-lr, axis=1, kind="stable")[:, :k]
    q = np.exp(np.take_along_axis(lr, order, axis=1)).astype(np.float32)
    gumbel = rng.gumbel(size=(n, vocab))
    sampled = np.argmax(lr + gumbel, axis=1)
    rollout_logp = lr[np.arange(n), sampled].astype(np.float32)
    rewards = (rng.random(n_resp) < 0.5).astype(np.float32)
    resp_idx = np.repeat(np.arange(n_resp), tokens)
    return dict(logits=z, head_ids=order.astype(np.int32), head_probs=q,
                sampled=sampled.astype(np.int32),
                rollout_logp=rollout_logp, resp_idx=resp_idx.astype(np.int32),
                rewards=rewards, group_size=group_size, n_responses=n_resp,
                temperature=float(temperature))


# --------------------------------------------------------------------------
# Large workloads (torch, any device; generated chunk by chunk)
# --------------------------------------------------------------------------
@dataclass
class BigSpec:
    """Generator parameters of one large workload."""
    vocab: int = VOCAB
    k: int = TOPK
    temperature: float = 1.0
    sd: float = 3.0          # std of the Gaussian part of the trainer logits
    zipf: float = 1.1        # exponent of the per-id Zipf bias
    noise: float = 0.1       # std of rollout - trainer logit noise
    seed: int = 1


def zipf_bias(spec, device):
    """b_v = -zipf * ln(rank_v) over a seeded permutation of 1..V (fp32)."""
    import torch
    g = torch.Generator(device="cpu").manual_seed(spec.seed * 1_000_003 + 7)
    rank = torch.randperm(spec.vocab, generator=g) + 1
    return (-spec.zipf * torch.log(rank.double())).float().to(device)


def _gen(device, seed):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def big_chunk(spec, rows, chunk_seed, device, bias=None, row_scale=None,
              out_of_head=None):
    """One chunk of ``rows`` positions of a large workload.

    row_scale: optional fp32 [rows] factor applied to the trainer logits
    before bf16 rounding (distribution stress classes).  out_of_head: optional
    bool [rows]; where set the sampled token is drawn from the rollout softmax
    restricted to the ids outside H, elsewhere restricted to H (when given).
    Returns a dict of tensors on ``device``.
    """
    import torch
    if bias is None:
        bias = zipf_bias(spec, device)
    g = _gen(device, chunk_seed)
    base = torch.randn(rows, spec.vocab, generator=g, device=device) * spec.sd
    base += bias
    if row_scale is not None:
        base *= row_scale.to(device)[:, None]
    z = base.to(torch.bfloat16)
    del base
    zr = z.float()
    zr += torch.randn(rows, spec.vocab, generator=g, device=device) * spec.noise
    zr /= spec.temperature
    lr = torch.log_softmax(zr, dim=1)
    del zr
    top_lp, head_ids = torch.topk(lr, spec.k, dim=1)
    head_probs = top_lp.exp()
    u = torch.rand(rows, spec.vocab, generator=g, device=device)
    u.clamp_(min=1e-30)
    gumbel = -torch.log(-torch.log(u))
    del u
    score = lr + gumbel
    del gumbel
    if out_of_head is not None:
        in_h = torch.zeros(rows, spec.vocab, dtype=torch.bool, device=device)
        in_h.scatter_(1, head_ids, True)
        ooh = out_of_head.to(device)[:, None]
        allowed = torch.where(ooh, ~in_h, in_h)
        score = score.masked_fill(~allowed, float("-inf"))
        del in_h, allowed
    sampled = torch.argmax(score, dim=1)
    del score
    rollout_logp = lr.gather(1, sampled[:, None])[:, 0]
    return dict(logits=z, head_ids=head_ids.to(torch.int32).contiguous(),
                head_probs=head_probs.float().contiguous(),
                sampled=sampled.to(torch.int32),
                rollout_logp=rollout_logp.float().contiguous())


def quick_check(device, seed=1, n_prompts=2, group_size=4, tokens=1024,
                spec=None, gen_rows=1024):
    """Quick-check workload: 2 x 4 x 1,024 = 8,192 positions, V = 248,320.

    Trainer logits bf16(N(0, 3^2) + Zipf(1.1) bias), rollout noise 0.1.
    Every position is valid; rewards Bernoulli(0.5) per response.
    """
    import torch
    spec = spec or BigSpec(seed=seed)
    n_resp = n_prompts * group_size
    n = n_resp * tokens
    bias = zipf_bias(spec, device)
    parts = [big_chunk(spec, min(gen_rows, n - r0), spec.seed * 7919 + r0,
                       device, bias=bias)
             for r0 in range(0, n, gen_rows)]
    out = {key: torch.cat([p[key] for p in parts]) for key in parts[0]}
    g = _gen("cpu", spec.seed * 31 + 5)
    out["rewards"] = (torch.rand(n_resp, generator=g) < 0.5).float().to(device)
    out["resp_idx"] = torch.arange(n_resp, dtype=torch.int32).repeat_interleave(
        tokens).to(device)
    out["group_size"] = group_size
    out["n_responses"] = n_resp
    out["temperature"] = spec.temperature
    return out


def full_step_lengths(seed=2, n_prompts=32, group_size=4, max_tokens=4096,
                      min_tokens=256):
    """Response lengths ~ UniformInt[256, 4096] for the full-step workload."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(min_tokens, max_tokens + 1,
                        size=n_prompts * group_size)


def full_step_chunk(device, chunk, lengths, chunk_rows=16_384, max_tokens=4096,
                    spec=None, gen_rows=1024):
    """Chunk ``chunk`` of the full-step workload (32 x 4 x 4,096 positions).

    Row r * 4096 + t belongs to response r; t >= length_r is padding
    (resp_idx = -1).  The logits generator is the tiny workload's
    distribution (N(0, 2^2), rollout noise 0.05) at V = 248,320 in bf16.
    """
    import torch
    spec = spec or BigSpec(sd=2.0, zipf=0.0, noise=0.05, seed=11)
    r0 = chunk * chunk_rows
    parts = [big_chunk(spec, gen_rows, spec.seed * 7919 + r0 + j, device)
             for j in range(0, chunk_rows, gen_rows)]
    out = {key: torch.cat([p[key] for p in parts]) for key in parts[0]}
    rows = torch.arange(r0, r0 + chunk_rows)
    resp = rows // max_tokens
    t = rows % max_tokens
    lens = torch.as_tensor(np.asarray(lengths))[resp]
    out["resp_idx"] = torch.where(t < lens, resp, -1).to(torch.int32).to(device)
    return out


def stress_chunk(device, chunk, sigma, chunk_rows=16_384, spec=None,
                 gen_rows=1024, seed=3):
    """Chunk of the distribution-stress workload at rollout noise ``sigma``.

    Row class i mod 3: peaked (logits x 8), flat (x 0.1), mixed (x s_i with
    s_i log-uniform in [0.1, 8]).  5% of rows draw the sampled token outside
    the recorded head, the rest inside it.
    """
    import torch
    spec = spec or BigSpec(noise=sigma, seed=seed + int(sigma * 1000))
    r0 = chunk * chunk_rows
    gcpu = _gen("cpu", spec.seed * 131 + chunk)
    rows = torch.arange(r0, r0 + chunk_rows)
    cls = rows % 3
    mixed = torch.exp(torch.empty(chunk_rows).uniform_(np.log(0.1), np.log(8.0),
                                                       generator=gcpu))
    scale = torch.where(cls == 0, torch.full_like(mixed, 8.0),
                        torch.where(cls == 1, torch.full_like(mixed, 0.1),
                                    mixed))
    ooh = torch.rand(chunk_rows, generator=gcpu) < 0.05
    bias = zipf_bias(spec, device)
    parts = []
    for j in range(0, chunk_rows, gen_rows):
        sl = slice(j, j + gen_rows)
        parts.append(big_chunk(spec, gen_rows, spec.seed * 7919 + r0 + j,
                               device, bias=bias, row_scale=scale[sl],
                               out_of_head=ooh[sl]))
    out = {key: torch.cat([p[key] for p in parts]) for key in parts[0]}
    out["resp_idx"] = torch.zeros(chunk_rows, dtype=torch.int32, device=device)
    return out


# --------------------------------------------------------------------------
# LM-head workload: hidden states and vocabulary projection (bf16)
# --------------------------------------------------------------------------
def lmhead_weights(device, vocab=VOCAB, d=4096, seed=5, w_sd=0.02, drift=1e-3):
    """Trainer vocabulary projection W = bf16(N(0, w_sd^2)) [vocab, d] and the
    rollout engine's copy bf16(W + N(0, drift^2)) (its weights differ slightly,
    as a low-precision rollout's do).  Logit std is about w_sd sqrt(d)."""
    import torch
    g = _gen(device, seed)
    w = torch.empty(vocab, d, device=device, dtype=torch.bfloat16)
    w_roll = torch.empty_like(w)
    step = 8192
    for r0 in range(0, vocab, step):
        x = torch.randn(min(step, vocab - r0), d, generator=g, device=device) * w_sd
        w[r0:r0 + x.shape[0]] = x.to(torch.bfloat16)
        x = w[r0:r0 + x.shape[0]].float()
        x += torch.randn(x.shape, generator=g, device=device) * drift
        w_roll[r0:r0 + x.shape[0]] = x.to(torch.bfloat16)
    return w, w_roll


def lmhead_chunk(device, w_roll, rows, seed, temperature=1.0, k=TOPK,
                 gen_rows=1024):
    """Rows of the LM-head workload: hidden states X = bf16(N(0, 1)) [rows, d]
    and the rollout's record (top-k ids and probabilities, sampled id and its
    log-probability) from the rollout logits X W_roll^T at ``temperature``."""
    import torch
    vocab, d = w_roll.shape
    g = _gen(device, seed)
    hidden = torch.randn(rows, d, generator=g, device=device).to(torch.bfloat16)
    wr = w_roll.float()
    ids, probs, samp, rlp = [], [], [], []
    for r0 in range(0, rows, gen_rows):
        x = hidden[r0:r0 + gen_rows].float()
        lr = torch.log_softmax((x @ wr.T) / temperature, dim=1)
        top_lp, top_id = torch.topk(lr, k, dim=1)
        u = torch.rand(lr.shape, generator=g, device=device).clamp_(min=1e-30)
        a = torch.argmax(lr - torch.log(-torch.log(u)), dim=1)
        ids.append(top_id.to(torch.int32))
        probs.append(top_lp.exp().float())
        samp.append(a.to(torch.int32))
        rlp.append(lr.gather(1, a[:, None])[:, 0].float())
        del lr, u
    del wr
    return dict(hidden=hidden, head_ids=torch.cat(ids).contiguous(),
                head_probs=torch.cat(probs).contiguous(),
                sampled=torch.cat(samp), rollout_logp=torch.cat(rlp).contiguous())
