"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/mfa.h, and rejects invalid calls on the host before any
HIP call (only failing validations are exercised here, so no kernel can
launch)."""

import os
import re

import pytest

from conftest import ROOT

# a missing or unloadable libmfa.so is a failure of this suite, not a skip
import decode_attention_attn_amd.mfa as mfa  # noqa: E402

FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first
MIS = 0x10001   # misaligned


def _declared():
    src = open(os.path.join(ROOT, "include", "mfa.h")).read()
    return sorted(set(re.findall(r"\b(mfa_[a-z_0-9]+)\s*\(", src)))


def test_header_symbols_are_exported():
    declared = _declared()
    assert set(declared) == set(mfa.EXPORTED)
    for name in declared:
        assert mfa.raw_function(name) is not None


def test_header_constants_match_the_binding():
    src = open(os.path.join(ROOT, "include", "mfa.h")).read()
    defs = dict(re.findall(r"#define\s+(MFA_[A-Z_]+)\s+(\d+)\s*$", src, re.M))
    assert int(defs["MFA_MAX_BATCH"]) == mfa.MFA_MAX_BATCH
    assert int(defs["MFA_MAX_TOKENS"]) == mfa.MFA_MAX_TOKENS


def test_version_and_status_strings():
    assert mfa.mfa_version() == 10000
    for code in (0, -1, -2, -3, -4, -5):
        assert mfa.mfa_status_string(code).startswith("MFA_")
    assert "unknown" in mfa.mfa_status_string(7)


def test_workspace_sizes():
    B, G = 32, 256
    assert mfa.mfa_decode_attn_workspace_size(B, G) == (G + B) * 64 * 256 * 4 + (G + B) * 64 * 4 + B * 8
    assert mfa.mfa_decode_attn_workspace_size(0, G) == 0
    assert mfa.mfa_decode_attn_workspace_size(B, -1) == 0
    for fn in (mfa.mfa_qproj_workspace_size, mfa.mfa_kv_append_workspace_size):
        for dt in (mfa.MFA_F32, mfa.MFA_BF16):
            assert fn(2, dt) > 0 and fn(128, dt) >= fn(2, dt)
        assert fn(2, mfa.MFA_FP8_E4M3) == 0
        assert fn(0, mfa.MFA_BF16) == 0
    assert mfa.mfa_oproj_workspace_size(2, mfa.MFA_F32) == 0


def _attn(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, off=FAKE, len=FAKE, scale=0.0625, ks=1.0, vs=1.0, out=FAKE, lse=None,
             ws=FAKE, ws_bytes=1 << 40, B=4, G=8, qdt=mfa.MFA_BF16, kvdt=mfa.MFA_BF16)
    a.update(kw)
    f = mfa.raw_function("mfa_decode_attn")
    return f(a["q"], a["k"], a["v"], a["off"], a["len"], a["scale"], a["ks"], a["vs"], a["out"], a["lse"], a["ws"],
             a["ws_bytes"], a["B"], a["G"], a["qdt"], a["kvdt"], None)


def test_decode_attn_rejects_bad_arguments():
    assert _attn(q=None) == mfa.MFA_ERR_INVALID_ARG
    assert _attn(len=None) == mfa.MFA_ERR_INVALID_ARG
    assert _attn(B=0) == mfa.MFA_ERR_INVALID_ARG
    assert _attn(B=mfa.MFA_MAX_BATCH + 1) == mfa.MFA_ERR_INVALID_ARG
    assert _attn(G=-1) == mfa.MFA_ERR_INVALID_ARG
    assert _attn(scale=float("nan")) == mfa.MFA_ERR_INVALID_ARG
    assert _attn(qdt=mfa.MFA_F32, kvdt=mfa.MFA_BF16) == mfa.MFA_ERR_UNSUPPORTED
    assert _attn(qdt=mfa.MFA_FP8_E4M3, kvdt=mfa.MFA_FP8_E4M3) == mfa.MFA_ERR_UNSUPPORTED
    assert _attn(qdt=7) == mfa.MFA_ERR_UNSUPPORTED
    assert _attn(k=MIS) == mfa.MFA_ERR_ALIGNMENT
    assert _attn(out=MIS) == mfa.MFA_ERR_ALIGNMENT
    assert _attn(off=FAKE + 4) == mfa.MFA_ERR_ALIGNMENT
    assert _attn(ws=None) == mfa.MFA_ERR_WORKSPACE
    need = mfa.mfa_decode_attn_workspace_size(4, 8)
    assert _attn(ws_bytes=need - 1) == mfa.MFA_ERR_WORKSPACE


def test_decode_attn_paged_rejects_bad_arguments():
    f = mfa.raw_function("mfa_decode_attn_paged")

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, table=FAKE, maxb=4, rows=64, len=FAKE, out=FAKE, ws=FAKE, nbytes=1 << 40,
                 B=4, G=8, qdt=mfa.MFA_BF16, kvdt=mfa.MFA_BF16)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["table"], a["maxb"], a["rows"], a["len"], 0.0625, 1.0, 1.0, a["out"],
                 None, a["ws"], a["nbytes"], a["B"], a["G"], a["qdt"], a["kvdt"], None)

    assert call(table=None) == mfa.MFA_ERR_INVALID_ARG
    assert call(maxb=0) == mfa.MFA_ERR_INVALID_ARG
    for rows in (0, 32, 96, 1 << 21):
        assert call(rows=rows) == mfa.MFA_ERR_INVALID_ARG, rows
    assert call(qdt=mfa.MFA_F32, kvdt=mfa.MFA_F32) == mfa.MFA_ERR_UNSUPPORTED
    assert call(table=FAKE + 2) == mfa.MFA_ERR_ALIGNMENT
    assert call(k=MIS) == mfa.MFA_ERR_ALIGNMENT
    assert call(ws=None) == mfa.MFA_ERR_WORKSPACE
    assert call(nbytes=mfa.mfa_decode_attn_workspace_size(4, 8) - 1) == mfa.MFA_ERR_WORKSPACE


def test_decode_attn_mt_rejects_bad_arguments():
    f = mfa.raw_function("mfa_decode_attn_mt")

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, off=FAKE, len=FAKE, n=2, out=FAKE, ws=FAKE, nbytes=1 << 40, B=4, G=8,
                 qdt=mfa.MFA_BF16, kvdt=mfa.MFA_BF16)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["off"], a["len"], a["n"], 0.0625, 1.0, 1.0, a["out"], None, a["ws"],
                 a["nbytes"], a["B"], a["G"], a["qdt"], a["kvdt"], None)

    for n in (0, -1, mfa.MFA_MAX_TOKENS + 1, 1 << 30):
        assert call(n=n) == mfa.MFA_ERR_INVALID_ARG, n
    assert call(off=None) == mfa.MFA_ERR_INVALID_ARG
    assert call(qdt=mfa.MFA_F32, kvdt=mfa.MFA_F32) == mfa.MFA_ERR_UNSUPPORTED
    assert call(q=MIS) == mfa.MFA_ERR_ALIGNMENT
    need = [mfa.mfa_decode_attn_mt_workspace_size(4, n, 8) for n in range(1, mfa.MFA_MAX_TOKENS + 1)]
    assert need[0] == mfa.mfa_decode_attn_workspace_size(4, 8)
    assert all(a < b for a, b in zip(need, need[1:])), need
    for n in (0, -1, mfa.MFA_MAX_TOKENS + 1):
        assert mfa.mfa_decode_attn_mt_workspace_size(4, n, 8) == 0, n
    for n in range(2, mfa.MFA_MAX_TOKENS + 1):
        assert call(n=n, nbytes=need[n - 1] - 1) == mfa.MFA_ERR_WORKSPACE, n


def test_decode_attn_paged_mt_rejects_bad_arguments():
    f = mfa.raw_function("mfa_decode_attn_paged_mt")

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, table=FAKE, maxb=4, rows=64, len=FAKE, n=2, out=FAKE, ws=FAKE,
                 nbytes=1 << 40, B=4, G=8, qdt=mfa.MFA_BF16, kvdt=mfa.MFA_FP8_E4M3)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["table"], a["maxb"], a["rows"], a["len"], a["n"], 0.0625, 1.0, 1.0,
                 a["out"], None, a["ws"], a["nbytes"], a["B"], a["G"], a["qdt"], a["kvdt"], None)

    assert call(table=None) == mfa.MFA_ERR_INVALID_ARG
    for n in (0, mfa.MFA_MAX_TOKENS + 1):
        assert call(n=n) == mfa.MFA_ERR_INVALID_ARG, n
    assert call(maxb=0) == mfa.MFA_ERR_INVALID_ARG
    assert call(rows=100) == mfa.MFA_ERR_INVALID_ARG
    assert call(qdt=mfa.MFA_F32, kvdt=mfa.MFA_F32) == mfa.MFA_ERR_UNSUPPORTED
    assert call(qdt=mfa.MFA_FP8_E4M3) == mfa.MFA_ERR_UNSUPPORTED
    assert call(len=FAKE + 2) == mfa.MFA_ERR_ALIGNMENT
    assert call(ws=None) == mfa.MFA_ERR_WORKSPACE
    for n in range(2, mfa.MFA_MAX_TOKENS + 1):
        assert call(n=n, nbytes=mfa.mfa_decode_attn_mt_workspace_size(4, n, 8) - 1) == mfa.MFA_ERR_WORKSPACE, n


def test_qproj_kv_append_rejects_bad_arguments():
    f = mfa.raw_function("mfa_qproj_kv_append")

    def call(**kw):
        a = dict(x=FAKE, wdq=FAKE, gamma=None, eps=1e-6, wuq=FAKE, wk=FAKE, wv=FAKE, q=FAKE, kc=FAKE, vc=FAKE,
                 off=FAKE, len=FAKE, lout=None, ks=1.0, vs=1.0, ws=FAKE, nbytes=1 << 40, B=4, cdt=mfa.MFA_BF16)
        a.update(kw)
        return f(a["x"], a["wdq"], a["gamma"], a["eps"], a["wuq"], a["wk"], a["wv"], a["q"], a["kc"], a["vc"],
                 a["off"], a["len"], a["lout"], a["ks"], a["vs"], a["ws"], a["nbytes"], a["B"], a["cdt"], None)

    need = mfa.mfa_qproj_kv_append_workspace_size(4)
    assert need > 0 and mfa.mfa_qproj_kv_append_workspace_size(0) == 0
    assert mfa.mfa_qproj_kv_append_workspace_size(mfa.MFA_MAX_BATCH + 1) == 0
    for k in ("x", "wdq", "wuq", "wk", "wv", "q", "kc", "vc", "off", "len"):
        assert call(**{k: None}) == mfa.MFA_ERR_INVALID_ARG, k
    assert call(B=0) == mfa.MFA_ERR_INVALID_ARG
    assert call(eps=-1.0) == mfa.MFA_ERR_INVALID_ARG
    assert call(cdt=mfa.MFA_F32) == mfa.MFA_ERR_UNSUPPORTED
    assert call(cdt=mfa.MFA_FP8_E4M3, ks=0.0) == mfa.MFA_ERR_INVALID_ARG
    assert call(cdt=mfa.MFA_FP8_E4M3, vs=float("inf")) == mfa.MFA_ERR_INVALID_ARG
    # a bf16 cache ignores the scales: validation goes on to the workspace check
    assert call(ks=0.0, nbytes=need - 1) == mfa.MFA_ERR_WORKSPACE
    assert call(x=MIS) == mfa.MFA_ERR_ALIGNMENT
    assert call(lout=FAKE + 2) == mfa.MFA_ERR_ALIGNMENT
    assert call(ws=None) == mfa.MFA_ERR_WORKSPACE
    assert call(nbytes=need - 1) == mfa.MFA_ERR_WORKSPACE


def test_projections_reject_bad_arguments():
    qp = mfa.raw_function("mfa_qproj")
    assert qp(None, FAKE, None, 1e-6, FAKE, FAKE, FAKE, 1 << 30, 2, mfa.MFA_F32, None) == mfa.MFA_ERR_INVALID_ARG
    assert qp(FAKE, FAKE, None, -1.0, FAKE, FAKE, FAKE, 1 << 30, 2, mfa.MFA_F32, None) == mfa.MFA_ERR_INVALID_ARG
    assert qp(FAKE, FAKE, None, 1e-6, FAKE, FAKE, FAKE, 1 << 30, 2, mfa.MFA_FP8_E4M3, None) == mfa.MFA_ERR_UNSUPPORTED
    assert qp(FAKE, MIS, None, 1e-6, FAKE, FAKE, FAKE, 1 << 30, 2, mfa.MFA_BF16, None) == mfa.MFA_ERR_ALIGNMENT
    need = mfa.mfa_qproj_workspace_size(2, mfa.MFA_BF16)
    assert qp(FAKE, FAKE, None, 1e-6, FAKE, FAKE, FAKE, need - 1, 2, mfa.MFA_BF16, None) == mfa.MFA_ERR_WORKSPACE
    kv = mfa.raw_function("mfa_kv_append")
    args = [FAKE] * 7 + [None, FAKE]  # x, w_k, w_v, k, v, off, len, len_out (none), ws
    assert kv(*args, 1 << 30, 2, mfa.MFA_BF16, mfa.MFA_FP8_E4M3, None) == mfa.MFA_ERR_UNSUPPORTED
    assert kv(*args, 1 << 30, 2, mfa.MFA_F32, mfa.MFA_BF16, None) == mfa.MFA_ERR_UNSUPPORTED
    assert kv(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, 1 << 30, 2, mfa.MFA_BF16, mfa.MFA_BF16,
              None) == mfa.MFA_ERR_INVALID_ARG
    assert kv(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 2, FAKE, 1 << 30, 2, mfa.MFA_BF16, mfa.MFA_BF16,
              None) == mfa.MFA_ERR_ALIGNMENT  # a misaligned seq_len_out
    assert kv(*args, 0, 2, mfa.MFA_BF16, mfa.MFA_BF16, None) == mfa.MFA_ERR_WORKSPACE
    k8 = mfa.raw_function("mfa_kv_append_fp8")
    ok = dict(sk=0.01, sv=0.02, ws=FAKE, nbytes=1 << 30, B=2, dt=mfa.MFA_BF16)

    def k8call(**kw):
        a = dict(ok, **kw)
        ptrs = [a.get(n, FAKE) for n in ("x", "wk", "wv", "kc", "vc", "off", "len")] + [a.get("lout")]
        return k8(*ptrs, a["sk"], a["sv"], a["ws"], a["nbytes"], a["B"], a["dt"], None)

    assert k8call(kc=None) == mfa.MFA_ERR_INVALID_ARG
    assert k8call(B=0) == mfa.MFA_ERR_INVALID_ARG
    for bad in (0.0, -1.0, float("nan"), float("inf"), 1e-45):
        assert k8call(sk=bad) == mfa.MFA_ERR_INVALID_ARG, bad
        assert k8call(sv=bad) == mfa.MFA_ERR_INVALID_ARG, bad
    assert k8call(dt=mfa.MFA_FP8_E4M3) == mfa.MFA_ERR_UNSUPPORTED
    assert k8call(vc=MIS) == mfa.MFA_ERR_ALIGNMENT
    assert k8call(off=FAKE + 4) == mfa.MFA_ERR_ALIGNMENT
    assert k8call(lout=FAKE + 2) == mfa.MFA_ERR_ALIGNMENT
    assert k8call(ws=None) == mfa.MFA_ERR_WORKSPACE
    assert k8call(nbytes=mfa.mfa_kv_append_workspace_size(2, mfa.MFA_BF16) - 1) == mfa.MFA_ERR_WORKSPACE
    op = mfa.raw_function("mfa_oproj")
    assert op(FAKE, FAKE, None, FAKE, 1 << 30, 2, mfa.MFA_BF16, None) == mfa.MFA_ERR_INVALID_ARG
    assert op(FAKE, FAKE, FAKE, FAKE, 1 << 30, 0, mfa.MFA_BF16, None) == mfa.MFA_ERR_INVALID_ARG
    assert op(FAKE, MIS, FAKE, FAKE, 1 << 30, 2, mfa.MFA_BF16, None) == mfa.MFA_ERR_ALIGNMENT
    need = mfa.mfa_oproj_workspace_size(128, mfa.MFA_BF16)
    if need > 0:
        assert op(FAKE, FAKE, FAKE, FAKE, need - 1, 128, mfa.MFA_BF16, None) == mfa.MFA_ERR_WORKSPACE


def test_block_fp8_projections_reject_bad_arguments():
    qp = mfa.raw_function("mfa_qproj_w8")

    def qcall(**kw):
        a = dict(dict(x=FAKE, wdq=FAKE, sdq=FAKE, g=None, eps=1e-6, wuq=FAKE, suq=FAKE, q=FAKE, ws=FAKE,
                      nbytes=1 << 30, B=2), **kw)
        return qp(a["x"], a["wdq"], a["sdq"], a["g"], a["eps"], a["wuq"], a["suq"], a["q"], a["ws"], a["nbytes"],
                  a["B"], None)

    for bad in (dict(sdq=None), dict(suq=None), dict(wuq=None), dict(B=0), dict(eps=-1.0), dict(eps=float("nan"))):
        assert qcall(**bad) == mfa.MFA_ERR_INVALID_ARG, bad
    assert qcall(sdq=FAKE + 2) == mfa.MFA_ERR_ALIGNMENT
    assert qcall(wdq=MIS) == mfa.MFA_ERR_ALIGNMENT
    assert qcall(ws=None) == mfa.MFA_ERR_WORKSPACE
    assert qcall(nbytes=mfa.mfa_qproj_workspace_size(2, mfa.MFA_BF16) - 1) == mfa.MFA_ERR_WORKSPACE
    kv = mfa.raw_function("mfa_kv_append_w8")

    def kcall(**kw):
        a = dict(dict(dt=mfa.MFA_FP8_E4M3, sk=0.01, sv=0.02, ws=FAKE, nbytes=1 << 30, B=2), **kw)
        ptrs = [a.get(n, FAKE) for n in ("x", "wk", "swk", "wv", "swv", "kc", "vc", "off", "len")] + [a.get("lout")]
        return kv(*ptrs, a["dt"], a["sk"], a["sv"], a["ws"], a["nbytes"], a["B"], None)

    assert kcall(swk=None) == mfa.MFA_ERR_INVALID_ARG
    assert kcall(swv=None) == mfa.MFA_ERR_INVALID_ARG
    assert kcall(B=mfa.MFA_MAX_BATCH + 1) == mfa.MFA_ERR_INVALID_ARG
    for bad in (0.0, -1.0, float("nan"), float("inf"), 1e-45):
        assert kcall(sk=bad) == mfa.MFA_ERR_INVALID_ARG, bad
        assert kcall(sv=bad) == mfa.MFA_ERR_INVALID_ARG, bad
    # the cache scales are not read for a bf16 cache
    assert kcall(dt=mfa.MFA_BF16, sk=0.0, ws=None) == mfa.MFA_ERR_WORKSPACE
    assert kcall(dt=mfa.MFA_F32) == mfa.MFA_ERR_UNSUPPORTED
    assert kcall(swv=FAKE + 1) == mfa.MFA_ERR_ALIGNMENT
    assert kcall(kc=MIS) == mfa.MFA_ERR_ALIGNMENT
    assert kcall(lout=FAKE + 1) == mfa.MFA_ERR_ALIGNMENT
    assert kcall(nbytes=mfa.mfa_kv_append_workspace_size(2, mfa.MFA_BF16) - 1) == mfa.MFA_ERR_WORKSPACE
    op = mfa.raw_function("mfa_oproj_w8")
    assert op(FAKE, FAKE, None, FAKE, FAKE, 1 << 30, 2, None) == mfa.MFA_ERR_INVALID_ARG
    assert op(FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, 0, None) == mfa.MFA_ERR_INVALID_ARG
    assert op(FAKE, FAKE, FAKE + 2, FAKE, FAKE, 1 << 30, 2, None) == mfa.MFA_ERR_ALIGNMENT
    assert op(FAKE, MIS, FAKE, FAKE, FAKE, 1 << 30, 2, None) == mfa.MFA_ERR_ALIGNMENT
    need = mfa.mfa_oproj_workspace_size(128, mfa.MFA_BF16)
    if need > 0:
        assert op(FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, 128, None) == mfa.MFA_ERR_WORKSPACE


def test_block_fp8_qproj_kv_append_rejects_bad_arguments():
    f = mfa.raw_function("mfa_qproj_kv_append_w8")

    def call(**kw):
        a = dict(x=FAKE, wdq=FAKE, sdq=FAKE, gamma=None, eps=1e-6, wuq=FAKE, suq=FAKE, wk=FAKE, sk=FAKE, wv=FAKE,
                 sv=FAKE, q=FAKE, kc=FAKE, vc=FAKE, off=FAKE, len=FAKE, lout=None, ks=1.0, vs=1.0, ws=FAKE,
                 nbytes=1 << 40, B=4, cdt=mfa.MFA_FP8_E4M3)
        a.update(kw)
        return f(a["x"], a["wdq"], a["sdq"], a["gamma"], a["eps"], a["wuq"], a["suq"], a["wk"], a["sk"], a["wv"],
                 a["sv"], a["q"], a["kc"], a["vc"], a["off"], a["len"], a["lout"], a["ks"], a["vs"], a["ws"],
                 a["nbytes"], a["B"], a["cdt"], None)

    need = mfa.mfa_qproj_kv_append_workspace_size(4)
    for k in ("x", "wdq", "sdq", "wuq", "suq", "wk", "sk", "wv", "sv", "q", "kc", "vc", "off", "len"):
        assert call(**{k: None}) == mfa.MFA_ERR_INVALID_ARG, k
    assert call(B=0) == mfa.MFA_ERR_INVALID_ARG
    assert call(B=mfa.MFA_MAX_BATCH + 1) == mfa.MFA_ERR_INVALID_ARG
    assert call(eps=float("nan")) == mfa.MFA_ERR_INVALID_ARG
    assert call(cdt=mfa.MFA_F32) == mfa.MFA_ERR_UNSUPPORTED
    for bad in (0.0, -1.0, float("nan"), float("inf"), 1e-45):
        assert call(ks=bad) == mfa.MFA_ERR_INVALID_ARG, bad
        assert call(vs=bad) == mfa.MFA_ERR_INVALID_ARG, bad
    # a bf16 cache ignores the cache scales
    assert call(cdt=mfa.MFA_BF16, ks=0.0, nbytes=need - 1) == mfa.MFA_ERR_WORKSPACE
    for k in ("sdq", "suq", "sk", "sv"):
        assert call(**{k: FAKE + 2}) == mfa.MFA_ERR_ALIGNMENT, k
    assert call(wk=MIS) == mfa.MFA_ERR_ALIGNMENT
    assert call(lout=FAKE + 2) == mfa.MFA_ERR_ALIGNMENT
    assert call(ws=None) == mfa.MFA_ERR_WORKSPACE
    assert call(nbytes=need - 1) == mfa.MFA_ERR_WORKSPACE


def test_bw_probe_rejects_bad_arguments():
    f = mfa.raw_function("mfa_bw_probe")
    assert f(None, 1024, FAKE, 8, None) == mfa.MFA_ERR_INVALID_ARG
    assert f(FAKE, 1024, None, 8, None) == mfa.MFA_ERR_INVALID_ARG
    for nbytes in (0, 8, 1000):
        assert f(FAKE, nbytes, FAKE, 8, None) == mfa.MFA_ERR_INVALID_ARG, nbytes
    for g in (-1, 65537):
        assert f(FAKE, 1024, FAKE, g, None) == mfa.MFA_ERR_INVALID_ARG, g
    assert f(MIS, 1024, FAKE, 8, None) == mfa.MFA_ERR_ALIGNMENT
    assert f(FAKE, 1024, FAKE + 2, 8, None) == mfa.MFA_ERR_ALIGNMENT


def test_single_hip_runtime_in_process():
    # libmfa must bind to the HIP runtime torch already loaded, not a second copy
    maps = open(f"/proc/{os.getpid()}/maps").read()
    runtimes = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(runtimes) == 1, runtimes
