"""Thin ctypes binding of libsc.so (the SC correction library for gfx950).

Argument marshalling only: every computation runs in the library's HIP
kernels.  Each function mirrors the C entry point of the same name in
``include/sc.h`` and launches on torch's current HIP stream.  Output buffers
are allocated with torch when not supplied.  A missing library is an error:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsc.so")

# Mirrors of the enums in include/sc.h
SC_OK, SC_ERR_ARG, SC_ERR_UNSUPPORTED, SC_ERR_HIP, SC_ERR_TOO_LARGE = 0, -1, -2, -3, -4
STATIC_SCRATCH_BYTES = 64 << 20
SC_F32, SC_BF16 = 0, 1
DEV_BAD_ID, DEV_DUP_ID, DEV_BAD_SAMPLED, DEV_NONFINITE, DEV_BAD_RESP = 1, 2, 4, 8, 16
ROW_DLOGITS, ROW_SCORE, ROW_CORRECTION = 0, 1, 2
IS_NONE, IS_TIS, IS_MIS = 0, 1, 2
STATS = ("lse", "logp_a", "tail", "P_H", "Q_H", "rho", "S", "loss", "tv", "kl",
         "k3", "entropy", "w", "weight", "rev_kl", "lse_lo")
NSTATS = len(STATS)
STAT = {name: i for i, name in enumerate(STATS)}
BATCH = ("sum_loss", "sum_k3", "sum_tv", "sum_kl", "sum_Q_H", "sum_P_H",
         "sum_entropy", "sum_rev_kl", "rows", "flagged", "max_w",
         "mean_loss", "mean_k3", "mean_tv", "mean_kl", "mean_Q_H", "mean_P_H",
         "mean_entropy", "mean_rev_kl")
NBATCH = len(BATCH)

_vp, _i64, _i32, _f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
_SIGS = {
    "sc_logprobs": [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _i32, _vp, _vp,
                    _f32, _vp, _vp, _vp, _vp, _vp],
    "sc_center": [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _vp, _i32, _vp,
                  _vp, _vp, _vp, _i32, _f32, _vp, _vp, _vp, _vp, _vp, _vp,
                  ctypes.c_int, _i64, ctypes.c_int, ctypes.c_int, _f32, _f32,
                  ctypes.c_int, _vp, _vp],
    "sc_correct": [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _vp, _i32, _vp,
                   _vp, _vp, _vp, _i32, _f32, _vp, _vp, _vp, _vp, _vp, _vp,
                   ctypes.c_int, _i64, ctypes.c_int, ctypes.c_int, _f32, _f32,
                  ctypes.c_int, _vp, _vp],
    "sc_group_norm": [_vp, _i32, _i32, _i32, _f32, _vp, _vp],
    "sc_count_valid": [_vp, _i64, _vp, _i32, _vp],
    "sc_batch_sums": [_vp, _vp, _i64, _vp, _vp, _i32, _vp],
    "sc_lmhead_workspace_size": [_i64, _i64, _i32],
    "sc_logprobs_lmhead": [_vp, _i64, _i32, _i64, _vp, _i64, _i64, _vp, _i32, _vp,
                           _vp, _f32, _vp, _vp, _vp, _vp, _i64, _vp, _vp],
    "sc_logprobs_lmhead_static": [_vp, _i64, _i32, _i64, _vp, _i64, _i64, _vp, _i32, _vp,
                                  _vp, _f32, _vp, _vp, _vp, _vp, _vp],
    "sc_lmhead_logits": [_vp, _i64, _i32, _i64, _vp, _i64, _i64, _vp, _i64, _vp],
    "sc_record": [_vp, ctypes.c_int, _i64, _i64, _i64, _f32, _i32, _vp, _vp, _vp, _vp,
                  _vp, _vp],
    "sc_lmhead_dlogits": [_vp, _i64, _i32, _i64, _vp, _i64, _i64, _vp, _vp, _i32, _vp, _vp,
                          _vp, _i32, _f32, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _i64, _vp],
    "sc_lmhead_backward_workspace_size": [_i64, _i64, _i32],
    "sc_lmhead_backward": [_vp, _i64, _i32, _i64, _vp, _i64, _i64, _vp, _vp, _i32, _vp, _vp,
                           _vp, _i32, _f32, _vp, _vp, _vp, _vp, ctypes.c_int, _vp,
                           ctypes.c_int, _i64, _vp, _i64, ctypes.c_int, _i64, _vp, _i64, _vp],
    "sc_reference_copy": [_vp, _vp, _i64, _vp],
    "sc_status_string": [ctypes.c_int],
    "sc_version": [],
}

_lib = None


class ScError(RuntimeError):
    """A non-zero sc_status returned by the library."""


def lib():
    """Load libsc.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "off_policy_logit_amd.build.build() (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = {"sc_status_string": ctypes.c_char_p,
                          "sc_lmhead_workspace_size": ctypes.c_int64,
                          "sc_lmhead_backward_workspace_size": ctypes.c_int64,
                          }.get(name, ctypes.c_int)
        _lib = L
    return _lib


def _check(status):
    if status != SC_OK:
        raise ScError(lib().sc_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return SC_BF16
    if t.dtype == torch.float32:
        return SC_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t, dtype, name):
    if t.dtype != dtype or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous {dtype} tensor")
    return t


def _rows(logits):
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise TypeError("logits must be [n_rows, vocab] with unit column stride")
    return logits.shape[0], logits.shape[1], logits.stride(0)


def _alloc_stats(n, k, device, head_logp=True):
    out = dict(
        row_stats=torch.empty(n, NSTATS, dtype=torch.float32, device=device),
        row_idx=torch.empty(n, 2, dtype=torch.int32, device=device))
    if head_logp:
        out["head_logp"] = torch.empty(n, k, dtype=torch.float32, device=device)
    return out


def logprobs(logits, head_ids, sampled, resp_idx=None, temperature=1.0,
             out=None, dev_status=None, stream=None):
    """sc_logprobs: lse, log p(a), tail mass, P_H, argmax, a_slot, log p at H."""
    n, V, stride = _rows(logits)
    k = head_ids.shape[1]
    _need(head_ids, torch.int32, "head_ids")
    _need(sampled, torch.int32, "sampled")
    if resp_idx is not None:
        _need(resp_idx, torch.int32, "resp_idx")
    out = out or _alloc_stats(n, k, logits.device)
    _check(lib().sc_logprobs(
        _ptr(logits), _dtype_code(logits), n, V, stride, _ptr(head_ids), k,
        _ptr(sampled), _ptr(resp_idx), float(temperature), _ptr(out["row_stats"]),
        _ptr(out["row_idx"]), _ptr(out.get("head_logp")), _ptr(dev_status),
        _stream(stream)))
    return out


def _default_hi(is_mode, is_hi):
    if is_hi is not None:
        return is_hi
    return 5.0 if is_mode == IS_MIS else 2.0


def _center_like(fn, logits, head_ids, head_probs, sampled, resp_idx,
                 advantages, temperature, n_valid, rollout_logp, out, row_out,
                 row_mode, coef, dev_status, stream, is_mode, is_lo, is_hi,
                 centering, vocab=None):
    if logits is not None:
        n, V, stride = _rows(logits)
        dcode = _dtype_code(logits)
    else:
        n, V, stride, dcode = head_ids.shape[0], vocab, vocab, SC_F32
    k = head_ids.shape[1]
    for t, dt, name in ((head_ids, torch.int32, "head_ids"),
                        (head_probs, torch.float32, "head_probs"),
                        (sampled, torch.int32, "sampled"),
                        (resp_idx, torch.int32, "resp_idx"),
                        (advantages, torch.float32, "advantages")):
        _need(t, dt, name)
    if row_out is not None:
        if row_out.dim() != 2 or row_out.stride(1) != 1:
            raise TypeError("row_out must be [n_rows, >= vocab] with unit column stride")
        ocode, ostride = _dtype_code(row_out), row_out.stride(0)
    else:
        ocode, ostride = SC_F32, 0
    _check(fn(
        _ptr(logits), dcode, n, V, stride, _ptr(head_ids), _ptr(head_probs), k,
        _ptr(sampled), _ptr(rollout_logp), _ptr(resp_idx), _ptr(advantages),
        advantages.shape[0], float(temperature), _ptr(n_valid),
        _ptr(out["row_stats"]), _ptr(out["row_idx"]), _ptr(out.get("head_logp")),
        _ptr(coef), _ptr(row_out), ocode, ostride, int(row_mode), int(is_mode),
        float(is_lo), float(_default_hi(is_mode, is_hi)), int(bool(centering)),
        _ptr(dev_status),
        _stream(stream)))


def center(stats, head_ids, head_probs, sampled, resp_idx, advantages,
           temperature=1.0, n_valid=None, rollout_logp=None, logits=None,
           row_out=None, row_mode=ROW_DLOGITS, coef=None, dev_status=None,
           stream=None, vocab=None, is_mode=IS_NONE, is_lo=0.5, is_hi=None,
           centering=True):
    """sc_center on the output dict of logprobs(); fills the remaining stats.

    is_mode / is_lo / is_hi select the importance weighting of the sampled
    token (IS_TIS: min(w, is_hi); IS_MIS: w inside [is_lo, is_hi], else 0;
    both need rollout_logp); is_hi defaults to 2.0 for TIS and 5.0 for MIS
    (the Score Centering page's settings table); centering=False drops the
    centering term."""
    if coef is None:
        coef = torch.empty_like(stats["head_logp"])
    if logits is None and vocab is None:
        raise TypeError("vocab is required when logits is None")
    _center_like(lib().sc_center, logits, head_ids, head_probs, sampled,
                 resp_idx, advantages, temperature, n_valid, rollout_logp,
                 stats, row_out, row_mode, coef, dev_status, stream, is_mode,
                 is_lo, is_hi, centering, vocab)
    stats["coef"] = coef
    return stats


def correct(logits, head_ids, head_probs, sampled, resp_idx, advantages,
            temperature=1.0, n_valid=None, rollout_logp=None, row_out=None,
            row_mode=ROW_DLOGITS, out=None, coef=None, dev_status=None,
            stream=None, is_mode=IS_NONE, is_lo=0.5, is_hi=None, centering=True):
    """sc_correct: every output of logprobs() and center() in one kernel."""
    n = logits.shape[0]
    k = head_ids.shape[1]
    out = out or _alloc_stats(n, k, logits.device)
    if coef is None:
        coef = torch.empty(n, k, dtype=torch.float32, device=logits.device)
    _center_like(lib().sc_correct, logits, head_ids, head_probs, sampled,
                 resp_idx, advantages, temperature, n_valid, rollout_logp, out,
                 row_out, row_mode, coef, dev_status, stream, is_mode, is_lo,
                 is_hi, centering)
    out["coef"] = coef
    return out


def group_norm(rewards, group_size, mode=0, eps=1e-6, out=None, stream=None):
    """sc_group_norm: advantages of consecutive groups of responses."""
    _need(rewards, torch.float32, "rewards")
    n = rewards.numel()
    if n % group_size:
        raise ValueError("rewards length must be a multiple of group_size")
    out = torch.empty_like(rewards) if out is None else out
    _check(lib().sc_group_norm(_ptr(rewards), n // group_size, group_size,
                               int(mode), float(eps), _ptr(out), _stream(stream)))
    return out


def count_valid(resp_idx, out=None, accumulate=False, stream=None):
    """sc_count_valid: exact int64 number of rows with resp_idx >= 0."""
    _need(resp_idx, torch.int32, "resp_idx")
    if out is None:
        out = torch.empty(1, dtype=torch.int64, device=resp_idx.device)
    _check(lib().sc_count_valid(_ptr(resp_idx), resp_idx.numel(), _ptr(out),
                                int(bool(accumulate)), _stream(stream)))
    return out


def batch_sums(row_stats, resp_idx, n_valid, out=None, accumulate=False,
               stream=None):
    """sc_batch_sums: float64 step sums and global-token means."""
    _need(row_stats, torch.float32, "row_stats")
    _need(resp_idx, torch.int32, "resp_idx")
    if out is None:
        out = torch.empty(NBATCH, dtype=torch.float64, device=row_stats.device)
    _check(lib().sc_batch_sums(_ptr(row_stats), _ptr(resp_idx), resp_idx.numel(),
                               _ptr(n_valid), _ptr(out), int(bool(accumulate)),
                               _stream(stream)))
    return out


def version():
    return lib().sc_version()


# ---------------------------------------------------------------------------
# Fused LM-head statistics
# ---------------------------------------------------------------------------
def lmhead_workspace_size(n_rows, vocab, k):
    """sc_lmhead_workspace_size: bytes of scratch sc_logprobs_lmhead needs."""
    size = lib().sc_lmhead_workspace_size(int(n_rows), int(vocab), int(k))
    if size < 0:
        _check(size)
    return size


def _bf16_matrix(t, name):
    if t.dtype != torch.bfloat16 or t.dim() != 2 or t.stride(1) != 1:
        raise TypeError(f"{name} must be a bf16 [rows, d] tensor with unit column stride")
    return t.shape[0], t.shape[1], t.stride(0)


def logprobs_lmhead(hidden, weight, head_ids, sampled, resp_idx=None,
                    temperature=1.0, out=None, workspace=None, dev_status=None,
                    stream=None):
    """sc_logprobs_lmhead: the outputs of logprobs() for logits hidden @ weight.T,
    without materialising the logits."""
    n, d, hs = _bf16_matrix(hidden, "hidden")
    V, dw, ws = _bf16_matrix(weight, "weight")
    if dw != d:
        raise ValueError("hidden and weight disagree on d")
    _need(head_ids, torch.int32, "head_ids")
    _need(sampled, torch.int32, "sampled")
    if resp_idx is not None:
        _need(resp_idx, torch.int32, "resp_idx")
    k = head_ids.shape[1]
    out = out or _alloc_stats(n, k, hidden.device)
    need = lmhead_workspace_size(n, V, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=hidden.device)
    _check(lib().sc_logprobs_lmhead(
        _ptr(hidden), n, d, hs, _ptr(weight), V, ws, _ptr(head_ids), k,
        _ptr(sampled), _ptr(resp_idx), float(temperature), _ptr(out["row_stats"]),
        _ptr(out["row_idx"]), _ptr(out.get("head_logp")), _ptr(workspace),
        workspace.numel(), _ptr(dev_status), _stream(stream)))
    return out


def logprobs_lmhead_static(hidden, weight, head_ids, sampled, resp_idx=None,
                           temperature=1.0, out=None, dev_status=None, stream=None):
    """sc_logprobs_lmhead_static: logprobs_lmhead() on the library's static
    per-GPU workspace; allocates nothing when `out` is given.  Calls that
    overlap on one GPU race."""
    n, d, hs = _bf16_matrix(hidden, "hidden")
    V, dw, ws = _bf16_matrix(weight, "weight")
    if dw != d:
        raise ValueError("hidden and weight disagree on d")
    _need(head_ids, torch.int32, "head_ids")
    _need(sampled, torch.int32, "sampled")
    if resp_idx is not None:
        _need(resp_idx, torch.int32, "resp_idx")
    k = head_ids.shape[1]
    out = out or _alloc_stats(n, k, hidden.device)
    _check(lib().sc_logprobs_lmhead_static(
        _ptr(hidden), n, d, hs, _ptr(weight), V, ws, _ptr(head_ids), k,
        _ptr(sampled), _ptr(resp_idx), float(temperature), _ptr(out["row_stats"]),
        _ptr(out["row_idx"]), _ptr(out.get("head_logp")), _ptr(dev_status),
        _stream(stream)))
    return out


def reference_copy(src, dst, stream=None):
    """sc_reference_copy: the streaming copy kernel used as the bandwidth
    reference (src and dst: contiguous device tensors of equal byte size)."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n or not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous and of equal byte size")
    _check(lib().sc_reference_copy(_ptr(src), _ptr(dst), n, _stream(stream)))
    return dst


def lmhead_logits(hidden, weight, out=None, stream=None):
    """sc_lmhead_logits: fp32 hidden @ weight.T from the fused kernel's GEMM."""
    n, d, hs = _bf16_matrix(hidden, "hidden")
    V, dw, ws = _bf16_matrix(weight, "weight")
    if dw != d:
        raise ValueError("hidden and weight disagree on d")
    if out is None:
        out = torch.empty(n, V, dtype=torch.float32, device=hidden.device)
    if out.dtype != torch.float32 or out.dim() != 2 or out.stride(1) != 1:
        raise TypeError("out must be a float32 [n, >= vocab] tensor with unit column stride")
    _check(lib().sc_lmhead_logits(_ptr(hidden), n, d, hs, _ptr(weight), V, ws,
                                  _ptr(out), out.stride(0), _stream(stream)))
    return out


def record(logits, k, sampled=None, temperature=1.0, head_ids=None, head_probs=None,
           sampled_logp=None, dev_status=None, stream=None):
    """sc_record: top-k candidate ids and probabilities of the rollout softmax
    per row (ties to the lower id), and the sampled token's log-probability."""
    n, V, stride = _rows(logits)
    if sampled is not None:
        _need(sampled, torch.int32, "sampled")
    dev = logits.device
    head_ids = torch.empty(n, k, dtype=torch.int32, device=dev) if head_ids is None else head_ids
    head_probs = torch.empty(n, k, dtype=torch.float32, device=dev) if head_probs is None else head_probs
    if sampled is not None and sampled_logp is None:
        sampled_logp = torch.empty(n, dtype=torch.float32, device=dev)
    _check(lib().sc_record(_ptr(logits), _dtype_code(logits), n, V, stride,
                           float(temperature), int(k), _ptr(sampled), _ptr(head_ids),
                           _ptr(head_probs), _ptr(sampled_logp), _ptr(dev_status),
                           _stream(stream)))
    return dict(head_ids=head_ids, head_probs=head_probs, sampled_logp=sampled_logp)


def _lm_dz_args(hidden, weight, stats, head_ids, head_probs, sampled, resp_idx,
                advantages, temperature, n_valid, centering):
    n, d, hs = _bf16_matrix(hidden, "hidden")
    V, dw, ws = _bf16_matrix(weight, "weight")
    if dw != d:
        raise ValueError("hidden and weight disagree on d")
    for t, dt, name in ((head_ids, torch.int32, "head_ids"),
                        (head_probs, torch.float32, "head_probs"),
                        (sampled, torch.int32, "sampled"),
                        (advantages, torch.float32, "advantages")):
        _need(t, dt, name)
    if resp_idx is not None:
        _need(resp_idx, torch.int32, "resp_idx")
    k = head_ids.shape[1]
    return [_ptr(hidden), n, d, hs, _ptr(weight), V, ws, _ptr(head_ids), _ptr(head_probs), k,
            _ptr(sampled), _ptr(resp_idx), _ptr(advantages), advantages.shape[0],
            float(temperature), _ptr(n_valid), _ptr(stats["row_stats"]),
            _ptr(stats["row_idx"]), _ptr(stats["head_logp"]), int(bool(centering))]


def lmhead_dlogits(hidden, weight, stats, head_ids, head_probs, sampled, resp_idx,
                   advantages, n_valid, temperature=1.0, centering=True, out=None,
                   stream=None):
    """sc_lmhead_dlogits: bf16 dLogits rows recomputed from hidden and weight;
    stats is the dict filled by logprobs_lmhead() then center()."""
    args = _lm_dz_args(hidden, weight, stats, head_ids, head_probs, sampled, resp_idx,
                       advantages, temperature, n_valid, centering)
    n, V = hidden.shape[0], weight.shape[0]
    if out is None:
        out = torch.empty(n, (V + 7) // 8 * 8, dtype=torch.bfloat16, device=hidden.device)[:, :V]
    _check(lib().sc_lmhead_dlogits(*args, _ptr(out), out.stride(0), _stream(stream)))
    return out


def lmhead_backward(hidden, weight, stats, head_ids, head_probs, sampled, resp_idx,
                    advantages, n_valid, temperature=1.0, centering=True, d_hidden=None,
                    d_weight=None, accumulate=False, chunk_rows=8192, workspace=None,
                    stream=None):
    """sc_lmhead_backward: (d_hidden, d_weight) of the step loss through the
    LM head, chunk_rows rows of dLogits at a time."""
    args = _lm_dz_args(hidden, weight, stats, head_ids, head_probs, sampled, resp_idx,
                       advantages, temperature, n_valid, centering)
    n, d = hidden.shape
    V = weight.shape[0]
    dev = hidden.device
    if d_hidden is None:
        d_hidden = torch.empty(n, d, dtype=torch.float32, device=dev)
    if d_weight is None:
        d_weight = torch.zeros(V, d, dtype=torch.float32, device=dev)
    need = lib().sc_lmhead_backward_workspace_size(int(chunk_rows), V, d)
    if need < 0:
        _check(need)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib().sc_lmhead_backward(
        *args, _ptr(d_hidden), _dtype_code(d_hidden), d_hidden.stride(0), _ptr(d_weight),
        d_weight.stride(0), int(bool(accumulate)), int(chunk_rows), _ptr(workspace),
        workspace.numel(), _stream(stream)))
    return d_hidden, d_weight
