"""The C-ABI library loads, exports every declared entry point and rejects bad
arguments before touching HIP (so these run on a host without a GPU)."""
import ctypes
import os
import re

import pytest

from off_policy_logit_amd import sc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: validation fails first
FAKE2 = ctypes.c_void_p(0x10002)     # 2-byte aligned only
FAKE1 = ctypes.c_void_p(0x10001)     # odd address
NULL = None
ARG, UNSUP, OK = sc.SC_ERR_ARG, sc.SC_ERR_UNSUPPORTED, sc.SC_OK


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(sc_\w+)\s*\(", text, re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"sc_logprobs", "sc_center", "sc_correct", "sc_group_norm",
            "sc_count_valid", "sc_batch_sums"} <= set(names)
    L = sc.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    L = sc.lib()
    for code in (OK, ARG, UNSUP, sc.SC_ERR_HIP, sc.SC_ERR_TOO_LARGE):
        assert L.sc_status_string(code).startswith(b"SC_")
    assert L.sc_version() >= 100


def logprobs(**kw):
    a = dict(logits=FAKE, dtype=sc.SC_BF16, n=4, V=1000, stride=1000, ids=FAKE,
             k=10, sampled=FAKE, resp=NULL, T=1.0, stats=FAKE, idx=FAKE,
             hlp=FAKE, dev=NULL, stream=NULL)
    a.update(kw)
    return sc.lib().sc_logprobs(a["logits"], a["dtype"], a["n"], a["V"], a["stride"],
                                a["ids"], a["k"], a["sampled"], a["resp"], a["T"],
                                a["stats"], a["idx"], a["hlp"], a["dev"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(logits=NULL), dict(ids=NULL), dict(sampled=NULL), dict(stats=NULL),
    dict(idx=NULL), dict(dtype=2), dict(dtype=-1), dict(n=-1), dict(V=0),
    dict(stride=999), dict(k=0), dict(k=1001), dict(k=1025, V=5000, stride=5000),
    dict(T=0.0), dict(T=-1.0), dict(T=float("nan")), dict(T=float("inf")),
    dict(logits=FAKE1), dict(dtype=sc.SC_F32, logits=FAKE2), dict(ids=FAKE2),
    dict(V=2 ** 31, stride=2 ** 31), dict(n=2 ** 31),
])
def test_logprobs_rejects_bad_arguments(kw):
    assert logprobs(**kw) == ARG


def test_logprobs_zero_rows_is_a_noop_without_hip():
    assert logprobs(n=0) == OK


def test_lds_limit_is_reported_as_unsupported():
    assert logprobs(V=2 ** 30, stride=2 ** 30, k=1024) == UNSUP
    assert logprobs(V=2 ** 24, stride=2 ** 24, k=1024) == UNSUP


def center(fn="sc_center", **kw):
    a = dict(logits=FAKE, dtype=sc.SC_BF16, n=4, V=1000, stride=1000, ids=FAKE,
             probs=FAKE, k=10, sampled=FAKE, rlp=NULL, resp=FAKE, adv=FAKE,
             nresp=2, T=1.0, nvalid=FAKE, stats=FAKE, idx=FAKE, hlp=FAKE,
             coef=FAKE, out=FAKE, odt=sc.SC_BF16, ostride=1000,
             mode=sc.ROW_DLOGITS, is_mode=sc.IS_NONE, lo=0.5, hi=2.0, cen=1,
             dev=NULL, stream=NULL)
    a.update(kw)
    return getattr(sc.lib(), fn)(
        a["logits"], a["dtype"], a["n"], a["V"], a["stride"], a["ids"], a["probs"],
        a["k"], a["sampled"], a["rlp"], a["resp"], a["adv"], a["nresp"], a["T"],
        a["nvalid"], a["stats"], a["idx"], a["hlp"], a["coef"], a["out"], a["odt"],
        a["ostride"], a["mode"], a["is_mode"], a["lo"], a["hi"], a["cen"],
        a["dev"], a["stream"])


@pytest.mark.parametrize("fn", ["sc_center", "sc_correct"])
@pytest.mark.parametrize("kw", [
    dict(probs=NULL), dict(resp=NULL), dict(adv=NULL), dict(nresp=-1),
    dict(mode=3), dict(mode=-1), dict(odt=5), dict(ostride=999),
    dict(nvalid=NULL), dict(out=FAKE1), dict(odt=sc.SC_F32, out=FAKE2),
    dict(logits=NULL), dict(T=0.0), dict(k=0), dict(coef=FAKE2),
    dict(is_mode=3), dict(is_mode=-1), dict(is_mode=sc.IS_TIS),
    dict(is_mode=sc.IS_MIS, rlp=FAKE, lo=2.0, hi=1.0),
    dict(is_mode=sc.IS_MIS, rlp=FAKE, lo=-0.1),
    dict(is_mode=sc.IS_TIS, rlp=FAKE, hi=0.0),
    dict(is_mode=sc.IS_TIS, rlp=FAKE, hi=float("inf")),
    dict(is_mode=sc.IS_MIS, rlp=FAKE, lo=float("nan")),
])
def test_center_and_correct_reject_bad_arguments(fn, kw):
    assert center(fn, **kw) == ARG


def test_center_without_row_out_needs_no_logits_or_n_valid():
    assert center(logits=NULL, out=NULL, nvalid=NULL, n=0) == OK
    assert center(logits=NULL, out=NULL, nvalid=NULL, hlp=NULL, n=0) == ARG
    # scores and corrections do not need N_valid
    assert center(nvalid=NULL, mode=sc.ROW_SCORE, n=0) == OK


def test_weighting_arguments_are_accepted():
    for is_mode in (sc.IS_TIS, sc.IS_MIS):
        assert center(is_mode=is_mode, rlp=FAKE, n=0) == OK
        assert center("sc_correct", is_mode=is_mode, rlp=FAKE, lo=0.0, hi=5.0, n=0) == OK
    # bounds are not read without weighting; centering off is always valid
    assert center(lo=float("nan"), hi=-1.0, cen=0, n=0) == OK


@pytest.mark.parametrize("args", [
    (NULL, 2, 4, 0, 1e-6, FAKE), (FAKE, 2, 4, 0, 1e-6, NULL), (FAKE, -1, 4, 0, 1e-6, FAKE),
    (FAKE, 2, 0, 0, 1e-6, FAKE), (FAKE, 2, 4097, 0, 1e-6, FAKE), (FAKE, 2, 4, 3, 1e-6, FAKE),
    (FAKE, 2, 4, 0, -1.0, FAKE), (FAKE, 2, 4, 0, float("nan"), FAKE), (FAKE2, 2, 4, 0, 0.0, FAKE),
])
def test_group_norm_rejects_bad_arguments(args):
    assert sc.lib().sc_group_norm(*args, NULL) == ARG


def test_group_norm_zero_groups_is_a_noop():
    assert sc.lib().sc_group_norm(FAKE, 0, 4, 0, 1e-6, FAKE, NULL) == OK


def test_count_and_batch_sums_reject_bad_arguments():
    L = sc.lib()
    assert L.sc_count_valid(FAKE, 10, NULL, 0, NULL) == ARG
    assert L.sc_count_valid(NULL, 10, FAKE, 0, NULL) == ARG
    assert L.sc_count_valid(FAKE, -1, FAKE, 0, NULL) == ARG
    assert L.sc_count_valid(FAKE, 10, FAKE2, 0, NULL) == ARG
    assert L.sc_batch_sums(FAKE, FAKE, 10, NULL, FAKE, 0, NULL) == ARG
    assert L.sc_batch_sums(FAKE, FAKE, 10, FAKE, NULL, 0, NULL) == ARG
    assert L.sc_batch_sums(NULL, FAKE, 10, FAKE, FAKE, 0, NULL) == ARG


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(sc, "_lib", None)
    monkeypatch.setattr(sc, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        sc.lib()


# --------------------------------------------------------------------------
# Fused LM-head entry points
# --------------------------------------------------------------------------
def test_lmhead_workspace_size():
    L = sc.lib()
    assert L.sc_lmhead_workspace_size(-1, 100, 4) == ARG
    assert L.sc_lmhead_workspace_size(10, 0, 1) == ARG
    assert L.sc_lmhead_workspace_size(10, 100, 0) == ARG
    assert L.sc_lmhead_workspace_size(10, 100, 101) == ARG
    assert L.sc_lmhead_workspace_size(0, 100, 4) >= 0
    small = L.sc_lmhead_workspace_size(1000, 4096, 128)
    big = L.sc_lmhead_workspace_size(2000, 4096, 128)
    # keys, recorded-id logits, per-split states and per-row scalars
    assert small >= 1000 * (128 * 12 + 16 * 16 + 16) and big > small


FAKE256 = ctypes.c_void_p(0x20000)


def lmhead(**kw):
    a = dict(x=FAKE, n=300, d=256, xs=256, w=FAKE, V=1000, ws=256, ids=FAKE, k=16,
             sampled=FAKE, resp=NULL, T=1.0, stats=FAKE, idx=FAKE, hlp=NULL,
             ws_ptr=FAKE256, ws_bytes=1 << 40, dev=NULL, stream=NULL)
    a.update(kw)
    return sc.lib().sc_logprobs_lmhead(
        a["x"], a["n"], a["d"], a["xs"], a["w"], a["V"], a["ws"], a["ids"], a["k"],
        a["sampled"], a["resp"], a["T"], a["stats"], a["idx"], a["hlp"], a["ws_ptr"],
        a["ws_bytes"], a["dev"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(x=NULL), dict(w=NULL), dict(ids=NULL), dict(sampled=NULL), dict(stats=NULL),
    dict(idx=NULL), dict(ws_ptr=NULL), dict(n=-1), dict(V=0), dict(d=0),
    dict(xs=255), dict(ws=200), dict(xs=260), dict(x=FAKE2), dict(w=FAKE1),
    dict(k=0), dict(k=1025, V=5000), dict(k=1001), dict(T=0.0), dict(T=float("inf")),
    dict(ws_bytes=100), dict(ws_ptr=ctypes.c_void_p(0x20010)), dict(xs=4194312, d=256),
])
def test_lmhead_rejects_bad_arguments(kw):
    assert lmhead(**kw) == ARG


def lmhead_static(**kw):
    a = dict(x=FAKE, n=300, d=256, xs=256, w=FAKE, V=1000, ws=256, ids=FAKE, k=16,
             sampled=FAKE, resp=NULL, T=1.0, stats=FAKE, idx=FAKE, hlp=NULL,
             dev=NULL, stream=NULL)
    a.update(kw)
    return sc.lib().sc_logprobs_lmhead_static(
        a["x"], a["n"], a["d"], a["xs"], a["w"], a["V"], a["ws"], a["ids"], a["k"],
        a["sampled"], a["resp"], a["T"], a["stats"], a["idx"], a["hlp"], a["dev"],
        a["stream"])


@pytest.mark.parametrize("kw", [
    dict(x=NULL), dict(w=NULL), dict(ids=NULL), dict(sampled=NULL), dict(stats=NULL),
    dict(idx=NULL), dict(n=-1), dict(V=0), dict(d=0), dict(xs=255), dict(x=FAKE2),
    dict(k=0), dict(k=1001), dict(T=0.0), dict(T=float("nan")),
])
def test_lmhead_static_rejects_bad_arguments(kw):
    assert lmhead_static(**kw) == ARG


def test_lmhead_static_limit_is_checked_before_any_hip_call():
    L = sc.lib()
    V, k = 248_320, 128
    lim = sc.STATIC_SCRATCH_BYTES
    assert L.sc_lmhead_workspace_size(11_881, V, k) <= lim
    assert L.sc_lmhead_workspace_size(11_882, V, k) > lim
    # Rejected on the host: no device is touched (there is none here).
    big = dict(n=11_882, d=4096, xs=4096, ws=4096, V=V, k=k)
    assert lmhead_static(**big) == sc.SC_ERR_TOO_LARGE
    assert lmhead_static(**dict(big, n=(1 << 31) - 1)) == sc.SC_ERR_TOO_LARGE
    assert b"static workspace" in L.sc_status_string(sc.SC_ERR_TOO_LARGE)
    assert lmhead_static(n=0) == OK
    assert lmhead_static(n=0, d=200, xs=200, ws=200) == UNSUP


def test_lmhead_d_must_be_a_multiple_of_64():
    assert lmhead(d=200, xs=200, ws=200) == UNSUP
    assert lmhead(n=0) == OK


def test_lmhead_logits_rejects_bad_arguments():
    L = sc.lib()
    f = L.sc_lmhead_logits
    assert f(FAKE, 10, 256, 256, FAKE, 100, 256, NULL, 100, NULL) == ARG
    assert f(FAKE, 10, 256, 256, FAKE, 100, 256, FAKE, 99, NULL) == ARG
    assert f(NULL, 10, 256, 256, FAKE, 100, 256, FAKE, 100, NULL) == ARG
    assert f(FAKE, 10, 100, 256, FAKE, 100, 256, FAKE, 100, NULL) == UNSUP
    assert f(FAKE, 0, 256, 256, FAKE, 100, 256, FAKE, 100, NULL) == OK


def record(**kw):
    a = dict(z=FAKE, dtype=sc.SC_BF16, n=4, V=1000, stride=1000, T=1.0, k=10, a=FAKE,
             ids=FAKE, probs=FAKE, lp=FAKE, dev=NULL, stream=NULL)
    a.update(kw)
    return sc.lib().sc_record(a["z"], a["dtype"], a["n"], a["V"], a["stride"], a["T"],
                              a["k"], a["a"], a["ids"], a["probs"], a["lp"], a["dev"],
                              a["stream"])


@pytest.mark.parametrize("kw", [
    dict(z=NULL), dict(ids=NULL), dict(probs=NULL), dict(dtype=3), dict(n=-1), dict(V=0),
    dict(stride=999), dict(k=0), dict(k=1001), dict(k=1025, V=5000, stride=5000),
    dict(T=0.0), dict(T=float("nan")), dict(a=NULL), dict(z=FAKE1), dict(ids=FAKE2),
])
def test_record_rejects_bad_arguments(kw):
    assert record(**kw) == ARG


def test_record_zero_rows_and_optional_sampled():
    assert record(n=0) == OK
    assert record(n=0, a=NULL, lp=NULL) == OK


def test_lmhead_backward_workspace_and_arguments():
    L = sc.lib()
    assert L.sc_lmhead_backward_workspace_size(0, 100, 64) == ARG
    assert L.sc_lmhead_backward_workspace_size(10, 0, 64) == ARG
    assert L.sc_lmhead_backward_workspace_size(10, 100, 0) == ARG
    # W^T [d, Vp] + dZ [chunk, Vp] + dZ^T [V, chunk_p] + X^T [d, chunk_p], bf16
    got = L.sc_lmhead_backward_workspace_size(100, 1000, 64)
    assert got >= 2 * (64 * 1024 + 100 * 1024 + 1000 * 128 + 64 * 128)

    def bwd(**kw):
        a = dict(x=FAKE, n=300, d=256, xs=256, w=FAKE, V=1000, ws=256, ids=FAKE, q=FAKE, k=16,
                 a=FAKE, resp=NULL, adv=FAKE, nresp=1, T=1.0, nv=FAKE, st=FAKE, idx=FAKE,
                 hlp=FAKE, cen=1, dh=FAKE, dhd=sc.SC_F32, dhs=256, dw=FAKE, dws=256, acc=0,
                 chunk=128, wsp=FAKE256, wsb=1 << 40, stream=NULL)
        a.update(kw)
        return L.sc_lmhead_backward(
            a["x"], a["n"], a["d"], a["xs"], a["w"], a["V"], a["ws"], a["ids"], a["q"], a["k"],
            a["a"], a["resp"], a["adv"], a["nresp"], a["T"], a["nv"], a["st"], a["idx"],
            a["hlp"], a["cen"], a["dh"], a["dhd"], a["dhs"], a["dw"], a["dws"], a["acc"],
            a["chunk"], a["wsp"], a["wsb"], a["stream"])
    assert bwd(n=0) == OK
    for kw in (dict(dh=NULL), dict(dw=NULL), dict(dhs=100), dict(dws=100), dict(chunk=0),
               dict(wsp=NULL), dict(wsb=1000), dict(st=NULL), dict(idx=NULL), dict(hlp=NULL),
               dict(adv=NULL), dict(nv=NULL), dict(dhd=7), dict(q=NULL)):
        assert bwd(**kw) == ARG, kw
    assert bwd(d=100, xs=104, ws=104) == UNSUP


def test_reference_copy_rejects_bad_arguments():
    L = sc.lib()
    assert L.sc_reference_copy(FAKE256, FAKE256, 0, NULL) == OK
    assert L.sc_reference_copy(NULL, FAKE256, 16, NULL) == ARG
    assert L.sc_reference_copy(FAKE256, NULL, 16, NULL) == ARG
    assert L.sc_reference_copy(FAKE256, FAKE256, 24, NULL) == ARG     # not a multiple of 16
    assert L.sc_reference_copy(FAKE256, FAKE256, -16, NULL) == ARG
    assert L.sc_reference_copy(FAKE2, FAKE256, 16, NULL) == ARG       # misaligned
    assert L.sc_reference_copy(FAKE256, FAKE256, (1 << 40) + 16, NULL) == ARG
