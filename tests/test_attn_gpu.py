"""GPU parity of mfa_decode_attn against the float64 oracle (needs an MI355X).

Small cases span several 32-row tiles, ragged tails, empty and length-1
sequences and every work split (one workgroup, odd counts, the default one per
CU); full-size cases use the benchmark's launch configuration (default split)
and compare every output element of every sequence.
"""

import numpy as np
import pytest

from parity import TOL, check, check_lse, passes

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from decode_attention_attn_amd import inputs as gen  # noqa: E402
from oracle import mfa_oracle as om  # noqa: E402

WL = {
    "bf16": gen.WORKLOADS["attn_bf16_4k"],
    "fp8_e4m3": gen.WORKLOADS["attn_fp8kv_4k"],
    "f32": gen.Workload("attn_f32", "attn", 8, 0, gen.F32, gen.F32),
}
LENGTHS = np.array([1, 31, 32, 33, 100, 257, 0, 700], dtype=np.int32)


def _runner():
    from decode_attention_attn_amd import runner  # fails loudly if libmfa.so is missing

    return runner


def _oracle(inp, ids=None):
    return om.decode_attn(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_off"], inp["seq_len"],
                          kind_q=inp["kind_q"], kind_kv=inp["kind_kv"], k_scale=inp["k_scale"],
                          v_scale=inp["v_scale"], batch_ids=ids)


def _make(kind, lengths=LENGTHS, seed=0):
    w = gen.scaled(WL[kind], batch=len(lengths), ctx=0, seed=seed)
    return gen.make_attn(w, lengths=np.asarray(lengths, dtype=np.int32))


@pytest.mark.parametrize("kind", ["bf16", "fp8_e4m3", "f32"])
@pytest.mark.parametrize("G", [1, 3, 64, 0])
def test_small_parity_all_splits(kind, G):
    r = _runner()
    print(f"[case] small {kind} G={G} lengths={LENGTHS.tolist()}", flush=True)
    inp = _make(kind)
    out, lse, _ = r.decode_attn(inp, num_workgroups=G)
    o_ref, l_ref = _oracle(inp)
    t = TOL[kind]
    check(f"out {kind} G={G}", r.to_f64(out), o_ref, t["atol"], t["rel"])
    check_lse(f"lse {kind} G={G}", r.to_f64(lse), l_ref, t["lse"])


@pytest.mark.parametrize("kind", ["bf16", "fp8_e4m3", "f32"])
def test_length_one_returns_v_row(kind):
    r = _runner()
    print(f"[case] L=1 {kind}", flush=True)
    inp = _make(kind, lengths=[1, 1, 1, 1, 1])
    out, lse, _ = r.decode_attn(inp)
    o_ref, l_ref = _oracle(inp)
    got = r.to_f64(out)
    if kind == "bf16":
        # p = 1 and l = 1 exactly, so the bf16 V row comes back bit for bit
        v = om.decode_bf16(inp["v_cache"])
        assert np.array_equal(got, np.repeat(v[:, None, :], 64, axis=1))
    elif kind == "f32":
        v = inp["v_cache"].astype(np.float64)
        assert np.array_equal(got, np.repeat(v[:, None, :], 64, axis=1))
    else:
        check("L=1 fp8", got, o_ref, 1e-2, 5e-3)
    check_lse(f"lse L=1 {kind}", r.to_f64(lse), l_ref, TOL[kind]["lse"])


def test_empty_sequences_give_zero_and_minus_inf():
    r = _runner()
    print("[case] empty sequences", flush=True)
    inp = _make("bf16", lengths=[0, 5, 0])
    out, lse, _ = r.decode_attn(inp)
    o = r.to_f64(out)
    lse = r.to_f64(lse)
    assert np.all(o[0] == 0) and np.all(o[2] == 0)
    assert np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[2])) and np.all(np.isfinite(lse[1]))


@pytest.mark.parametrize("G", [3, 0])
def test_empty_sequences_beyond_the_first_64(G):
    # empties among the first 64 sequences and after them take different paths
    r = _runner()
    lengths = np.full(70, 5, dtype=np.int32)
    lengths[[0, 2, 63, 64, 69]] = 0
    lengths[[1, 65]] = 300
    print(f"[case] 70 sequences with empties, G={G}", flush=True)
    inp = _make("bf16", lengths=lengths)
    out, lse, _ = r.decode_attn(inp, num_workgroups=G)
    o_ref, l_ref = _oracle(inp)
    check(f"out empties G={G}", r.to_f64(out), o_ref, 2e-2, 1e-2)
    check_lse(f"lse empties G={G}", r.to_f64(lse), l_ref, 2e-3)


def test_workspace_reuse_across_batch_sizes():
    # one workspace, calls of different sizes in turn: results must not
    # depend on what ran before in it, and repeat bit for bit
    r = _runner()
    print("[case] workspace reuse across batch sizes", flush=True)
    inp_a = _make("bf16", lengths=[3000, 17, 1500, 4096])
    inp_b = _make("bf16", lengths=LENGTHS, seed=1)
    call_a = r.AttnCall(r.upload_attn(inp_a))
    call_b = r.AttnCall(r.upload_attn(inp_b))
    assert call_b.ws.numel() >= call_a.ws.numel()
    call_a.ws = call_b.ws
    outs = []
    for call in (call_a, call_b, call_a, call_b):
        o, l = call()
        torch.cuda.synchronize()
        outs.append((r.to_f64(o), r.to_f64(l)))
    for (o, l), inp in zip(outs[:2], (inp_a, inp_b)):
        o_ref, l_ref = _oracle(inp)
        check("reused workspace out", o, o_ref, 2e-2, 1e-2)
        check_lse("reused workspace lse", l, l_ref, 2e-3)
    for i in (0, 1):
        assert np.array_equal(outs[i][0], outs[i + 2][0]) and np.array_equal(outs[i][1], outs[i + 2][1])


@pytest.mark.parametrize("kind", ["bf16", "fp8_e4m3"])
def test_splits_agree_and_repeat_bitwise(kind):
    r = _runner()
    print(f"[case] split agreement / determinism {kind}", flush=True)
    inp = _make(kind, lengths=[3000, 17, 1500, 4096])
    outs = {}
    for G in (1, 5, 37, 0):
        o, _, _ = r.decode_attn(inp, num_workgroups=G)
        outs[G] = r.to_f64(o)
    for G in (5, 37, 0):
        check(f"G=1 vs G={G}", outs[G], outs[1], 2e-2, 1e-2)
    o2, _, _ = r.decode_attn(inp, num_workgroups=37)
    assert np.array_equal(r.to_f64(o2), outs[37])


def test_uniform_scores_and_unit_values():
    r = _runner()
    print("[case] constant K / V = 1", flush=True)
    inp = _make("bf16", lengths=[200, 77])
    rows = int(inp["seq_len"].sum())
    inp_k = dict(inp, k_cache=np.repeat(inp["k_cache"][:1], rows, axis=0))
    out, _, _ = r.decode_attn(inp_k)
    v = om.decode_bf16(inp["v_cache"])
    mean = np.stack([np.broadcast_to(v[0:200].mean(0), (64, 256)), np.broadcast_to(v[200:277].mean(0), (64, 256))])
    check("constant K -> mean of V", r.to_f64(out), mean, 2e-2, 1e-2)
    one = gen.f32_to_bf16_bits(np.ones((rows, 256), dtype=np.float32))
    out, _, _ = r.decode_attn(dict(inp, v_cache=one))
    assert np.max(np.abs(r.to_f64(out) - 1.0)) < 4e-3


def test_large_score_offset_is_stable():
    # K + c with q.c/16 ~ 1e3: exp overflows in fp32 unless the running max is subtracted
    r = _runner()
    print("[case] large score offset", flush=True)
    inp = _make("bf16", lengths=[300, 64])
    q = om.decode_bf16(inp["q"])
    c = q[0].sum(axis=0)
    c = (c / np.linalg.norm(c) * 1000.0).astype(np.float32)
    k = (om.decode_bf16(inp["k_cache"]) + c).astype(np.float32)
    inp2 = dict(inp, k_cache=gen.f32_to_bf16_bits(k))
    out, lse, _ = r.decode_attn(inp2)
    o_ref, l_ref = _oracle(inp2)
    check("offset out", r.to_f64(out), o_ref, 2e-2, 1e-2)
    assert np.all(np.isfinite(r.to_f64(lse)))


def test_negative_controls_fail_the_gate():
    r = _runner()
    print("[case] negative controls", flush=True)
    inp = _make("bf16", lengths=[4096, 4096, 4096])
    out, _, _ = r.decode_attn(inp)
    got = r.to_f64(out)
    o_ref, _ = _oracle(inp)
    t = TOL["bf16"]
    assert passes(got, o_ref, t["atol"], t["rel"])
    assert not passes(np.zeros_like(got), o_ref, t["atol"], t["rel"])
    assert not passes(np.roll(got, 1, axis=1), o_ref, t["atol"], t["rel"])
    half = dict(inp, seq_len=inp["seq_len"] // 2)
    o_half, _ = _oracle(half)
    assert not passes(got, o_half, t["atol"], t["rel"])
    # one row too few is visible at short length
    inp16 = _make("bf16", lengths=[16, 16, 16])
    out16, _, _ = r.decode_attn(inp16)
    o_ok, _ = _oracle(inp16)
    o_short, _ = _oracle(dict(inp16, seq_len=inp16["seq_len"] - 1))
    assert passes(r.to_f64(out16), o_ok, t["atol"], t["rel"])
    assert not passes(r.to_f64(out16), o_short, t["atol"], t["rel"])


def _full(name):
    r = _runner()
    w = gen.WORKLOADS[name]
    print(f"[case] full {name}, every sequence", flush=True)
    inp = gen.make_attn(w)
    out, lse, _ = r.decode_attn(inp)
    got = r.to_f64(out)
    gl = r.to_f64(lse)
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(gl))
    o_ref, l_ref = _oracle(inp)
    t = TOL[w.kv]
    check(f"{name} out (all {len(got)} sequences)", got, o_ref, t["atol"], t["rel"])
    check_lse(f"{name} lse (all sequences)", gl, l_ref, t["lse"])
    # each sequence on its own too: a wrong piece of one sequence cannot hide
    # in the batch-wide relative error
    for b in range(len(got)):
        check(f"{name} out[{b}]", got[b], o_ref[b], t["atol"], t["rel"], quiet=True)
    return inp


def test_full_attn_bf16_4k():
    _full("attn_bf16_4k")


def test_full_attn_fp8kv_4k():
    _full("attn_fp8kv_4k")


def test_full_attn_bf16_ragged():
    _full("attn_bf16_ragged")


# ------------------------------------------------------------------ extremes
@pytest.mark.parametrize("kind", ["bf16", "fp8_e4m3"])
def test_single_long_sequence(kind):
    # one sequence of 256K keys: every workgroup takes a piece of it and the
    # combine merges one partial per workgroup (batches of 8, many rounds)
    r = _runner()
    print(f"[case] one sequence of 262144 keys, {kind}", flush=True)
    inp = _make(kind, lengths=[262144], seed=5)
    out, lse, _ = r.decode_attn(inp)
    o_ref, l_ref = _oracle(inp)
    t = TOL[kind]
    check(f"long sequence out {kind}", r.to_f64(out), o_ref, t["atol"], t["rel"])
    check_lse(f"long sequence lse {kind}", r.to_f64(lse), l_ref, t["lse"])


def test_many_short_sequences():
    # 4096 sequences of 0..40 keys: each workgroup walks across many whole
    # sequences (every tile is a sequence's tail)
    r = _runner()
    lengths = np.random.default_rng(11).integers(0, 41, size=4096).astype(np.int32)
    print(f"[case] 4096 sequences of 0..40 keys ({int((lengths == 0).sum())} empty)", flush=True)
    inp = _make("bf16", lengths=lengths, seed=6)
    out, lse, _ = r.decode_attn(inp)
    o_ref, l_ref = _oracle(inp)
    check("many short out", r.to_f64(out), o_ref, 2e-2, 1e-2)
    check_lse("many short lse", r.to_f64(lse), l_ref, 2e-3)


def test_maximum_batch():
    # B = MFA_MAX_BATCH (65536): mostly one key per sequence (the output is
    # then that V row bit for bit), a few longer and empty ones checked
    # against the oracle
    r = _runner()
    B = 65536
    lengths = np.ones(B, dtype=np.int32)
    lengths[::4096] = 37
    lengths[[5, 40000]] = 0
    lengths[-1] = 300
    print(f"[case] maximum batch B={B}", flush=True)
    inp = _make("bf16", lengths=lengths, seed=7)
    dev = r.upload_attn(inp)
    out, lse = r.AttnCall(dev)()
    torch.cuda.synchronize()
    one = torch.as_tensor(np.nonzero(lengths == 1)[0], device=out.device)
    rows = dev["off"][one]
    want = dev["v"][rows].unsqueeze(1).expand(-1, 64, -1)
    assert torch.equal(out[one], want), "L = 1 sequences must return their V row exactly"
    ids = [0, 4096, 5, 40000, 65535, 12345]
    o_ref, l_ref = _oracle(inp, ids)
    check("maximum batch out", r.to_f64(out[ids]), o_ref, 2e-2, 1e-2)
    check_lse("maximum batch lse", r.to_f64(lse[ids]), l_ref, 2e-3)
