"""GPU parity of the whole decode step (mfa_qproj, mfa_kv_append,
mfa_decode_attn, mfa_oproj) against the float64 oracle (needs an MI355X).

Checked per stage: q, the appended K/V rows (and that no other cache byte
changed), the attention output and lse, and y. "End to end" compares with the
oracle run from the stored inputs alone; "stage isolated" feeds the oracle's
attention the GPU's own q and cache, so each kernel's error is seen alone.
"""

import dataclasses
import math

import numpy as np
import pytest

from parity import TOL, check, check_lse

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from decode_attention_attn_amd import inputs as gen  # noqa: E402
from oracle import mfa_oracle as om  # noqa: E402


def _run_layer(inp, num_workgroups=0, fused=True):
    from decode_attention_attn_amd import runner

    dev = runner.upload_layer(inp)
    k_before = dev["k"].clone()
    v_before = dev["v"].clone()
    call = runner.LayerCall(dev, num_workgroups, fused_q_kv=fused)
    call()
    torch.cuda.synchronize()
    return runner, dev, call, k_before, v_before


def _stage_isolated_attn(runner, dev, call, inp, ids, chunk=16):
    """Oracle attention fed the GPU's own q and cache rows (sequences ``ids``,
    ``chunk`` at a time, so only that many sequences' rows sit on the host)."""
    outs, lses = [], []
    for c0 in range(0, len(ids), chunk):
        part = list(ids[c0:c0 + chunk])
        lens = inp["seq_len"][part] + 1
        sel = torch.cat([torch.arange(int(inp["seq_off"][b]), int(inp["seq_off"][b]) + int(n),
                                      device=dev["k"].device) for b, n in zip(part, lens)])
        offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
        o, lse = om.decode_attn(runner.to_f64(call.q[torch.as_tensor(part, device=call.q.device)]),
                                runner.to_f64(dev["k"][sel]), runner.to_f64(dev["v"][sel]), offs, lens)
        outs.append(o)
        lses.append(lse)
    return np.concatenate(outs), np.concatenate(lses)


def _check_layer(inp, kind, ids=None, num_workgroups=0, fused=True):
    """Every output of the sequences ``ids`` (all of them by default)."""
    runner, dev, call, k_before, v_before = _run_layer(inp, num_workgroups, fused)
    # the append hands attention the length including the new row
    assert torch.equal(call.len_after, dev["len"] + 1)
    t = TOL[kind]
    B = len(inp["seq_len"])
    ids = list(range(B)) if ids is None else list(ids)
    ref = om.decode_layer(inp, batch_ids=ids)
    rows = (inp["seq_off"] + inp["seq_len"]).astype(np.int64)
    check(f"{kind} q", runner.to_f64(call.q)[ids], ref["q"], t["atol"], t["rel"])
    k_new = runner.to_f64(dev["k"][torch.as_tensor(rows[ids], device=dev["k"].device)])
    v_new = runner.to_f64(dev["v"][torch.as_tensor(rows[ids], device=dev["v"].device)])
    check(f"{kind} k_new", k_new, ref["k_new"], t["atol"], t["rel"])
    check(f"{kind} v_new", v_new, ref["v_new"], t["atol"], t["rel"])
    # no other cache row changed
    mask = torch.ones(dev["k"].shape[0], dtype=torch.bool, device=dev["k"].device)
    mask[torch.as_tensor(rows, device=mask.device)] = False
    assert torch.equal(dev["k"][mask], k_before[mask]) and torch.equal(dev["v"][mask], v_before[mask])
    # attention and output, end to end
    o_got = runner.to_f64(call.o)[ids]
    check(f"{kind} o (end to end, {len(ids)} sequences)", o_got, ref["o"], t["atol"], t["rel"])
    for i, b in enumerate(ids):
        check(f"{kind} o[{b}] (end to end)", o_got[i], ref["o"][i], t["atol"], t["rel"], quiet=True)
    check_lse(f"{kind} lse (end to end)", runner.to_f64(call.lse)[ids], ref["lse"], max(t["lse"], 5e-3))
    check(f"{kind} y (end to end)", runner.to_f64(call.y)[ids], ref["y"], t["atol"], t["rel"])
    # stage isolated: oracle attention on the GPU's q and cache, oracle y on the GPU's o
    o_iso, _ = _stage_isolated_attn(runner, dev, call, inp, ids)
    check(f"{kind} o (stage isolated)", o_got, o_iso, t["atol"], t["rel"])
    y_iso = om.out_proj(o_got, _w_o(inp))
    check(f"{kind} y (stage isolated)", runner.to_f64(call.y)[ids], y_iso, t["atol"], t["rel"])
    return runner, dev, call, ref


def _w_o(inp):
    if inp.get("kind_w") == gen.FP8_BLOCK:
        return om.dequantize_blocks_e4m3fn(inp["w_o"], inp["w_o_scale"])
    return om.to_f64(inp["w_o"], inp["kind_act"])


def test_layer_tiny_fp32_full():
    print("[case] layer tiny_fp32 (full size)", flush=True)
    inp = gen.make_layer(gen.WORKLOADS["tiny_fp32"])
    _check_layer(inp, "f32")


@pytest.mark.parametrize("G", [0, 3])
def test_layer_bf16_small(G):
    print(f"[case] layer bf16 small B=5 ctx=300 G={G}", flush=True)
    w = gen.scaled(gen.WORKLOADS["layer_bf16_8k"], batch=5, ctx=300)
    inp = gen.make_layer(w)
    _check_layer(inp, "bf16", num_workgroups=G)


@pytest.mark.parametrize("B", [1, 200])
def test_layer_bf16_batch_edges(B):
    # one sequence; and more sequences than one 128-row GEMM tile (a second,
    # partly filled batch chunk in every projection)
    print(f"[case] layer bf16 B={B} ctx=64", flush=True)
    w = gen.scaled(gen.WORKLOADS["layer_bf16_8k"], batch=B, ctx=64)
    inp = gen.make_layer(w)
    _check_layer(inp, "bf16")


def test_layer_maximum_batch():
    # B = MFA_MAX_BATCH (65536) sequences of one cached row: 512 batch chunks
    # in every projection; sampled sequences against the oracle (indexed on
    # the device, so nothing of full size is converted on the host)
    B = 65536
    print(f"[case] layer bf16 maximum batch B={B} ctx=1", flush=True)
    inp = gen.make_layer(gen.scaled(gen.WORKLOADS["layer_bf16_8k"], batch=B, ctx=1))
    runner, dev, call, k_before, v_before = _run_layer(inp)
    ids = [0, 1, 40000, 65535]
    ref = om.decode_layer(inp, batch_ids=ids)
    t = TOL["bf16"]
    sel = torch.as_tensor(ids, device=dev["x"].device)
    rows = torch.as_tensor((inp["seq_off"] + inp["seq_len"])[ids].astype(np.int64), device=dev["k"].device)
    check("max batch q", runner.to_f64(call.q[sel]), ref["q"], t["atol"], t["rel"])
    check("max batch k_new", runner.to_f64(dev["k"][rows]), ref["k_new"], t["atol"], t["rel"])
    check("max batch v_new", runner.to_f64(dev["v"][rows]), ref["v_new"], t["atol"], t["rel"])
    check("max batch o", runner.to_f64(call.o[sel]), ref["o"], t["atol"], t["rel"])
    # two keys per sequence: the lse follows two single scores, each carrying
    # the bf16 rounding of q and of the new K row (nothing averages out), so
    # end to end it is held to the bf16 output tolerance; stage isolated
    # (oracle attention on the GPU's own q and cache rows) to the lse one
    check_lse("max batch lse (end to end)", runner.to_f64(call.lse[sel]), ref["lse"], t["atol"])
    lens = inp["seq_len"][ids] + 1
    span = torch.cat([torch.arange(int(inp["seq_off"][b]), int(inp["seq_off"][b]) + int(n), device=dev["k"].device)
                      for b, n in zip(ids, lens)])
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    o_iso, l_iso = om.decode_attn(runner.to_f64(call.q[sel]), runner.to_f64(dev["k"][span]),
                                  runner.to_f64(dev["v"][span]), offs, lens)
    check("max batch o (stage isolated)", runner.to_f64(call.o[sel]), o_iso, t["atol"], t["rel"])
    check_lse("max batch lse (stage isolated)", runner.to_f64(call.lse[sel]), l_iso, t["lse"])
    check("max batch y", runner.to_f64(call.y[sel]), ref["y"], t["atol"], t["rel"])
    # the cached row of every sequence is untouched
    cached = torch.as_tensor(inp["seq_off"].astype(np.int64), device=dev["k"].device)
    assert torch.equal(dev["k"][cached], k_before[cached]) and torch.equal(dev["v"][cached], v_before[cached])


def test_layer_bf16_8k_full():
    print("[case] layer layer_bf16_8k (full size, every sequence)", flush=True)
    inp = gen.make_layer(gen.WORKLOADS["layer_bf16_8k"])
    _check_layer(inp, "bf16")


# ------------------------------------------------------------------ e4m3 cache (quantize on append)
def _check_codes(name, got, want, exact, scale):
    """Appended e4m3 bytes against the oracle's. The GPU rounds its fp32
    projection, the oracle the exact one, so a code may differ where the exact
    value sits at a rounding midpoint; there the GPU's code must be as close to
    the exact value as the oracle's, up to the fp32 accumulation error."""
    t = om.e4m3fn_table()
    got, want = np.asarray(got, dtype=np.uint8), np.asarray(want, dtype=np.uint8)
    assert np.all(np.isfinite(t[got])), f"{name}: NaN code written"
    same = got == want
    y = np.asarray(exact, dtype=np.float64) / float(np.float32(scale))
    dg, dw = np.abs(t[got] - y), np.abs(t[want] - y)
    bad = ~same & (dg > dw + 1e-4 * np.abs(y) + 1e-6)
    print(f"[parity] {name}: {int((~same).sum())} of {got.size} codes differ (all at rounding midpoints: "
          f"{not bool(bad.any())})", flush=True)
    assert not bad.any(), f"{name}: {int(bad.sum())} codes farther from the exact value than the oracle's"
    assert same.mean() >= 0.99, f"{name}: only {same.mean():.4f} of the codes agree"


def _check_layer_fp8(inp, ids=None, num_workgroups=0, fused=True):
    runner, dev, call, k_before, v_before = _run_layer(inp, num_workgroups, fused)
    t, tb = TOL["fp8_e4m3"], TOL["bf16"]
    ids = list(range(len(inp["seq_len"]))) if ids is None else list(ids)
    ref = om.decode_layer(inp, batch_ids=ids)
    rows = (inp["seq_off"] + inp["seq_len"]).astype(np.int64)
    sel = torch.as_tensor(rows[ids], device=dev["k"].device)
    check("fp8 layer q", runner.to_f64(call.q)[ids], ref["q"], tb["atol"], tb["rel"])
    _check_codes("fp8 layer k_new", dev["k"][sel].cpu().numpy(), ref["k_new_codes"], ref["k_new"], inp["k_scale"])
    _check_codes("fp8 layer v_new", dev["v"][sel].cpu().numpy(), ref["v_new_codes"], ref["v_new"], inp["v_scale"])
    # no other cache byte changed
    mask = torch.ones(dev["k"].shape[0], dtype=torch.bool, device=dev["k"].device)
    mask[torch.as_tensor(rows, device=mask.device)] = False
    assert torch.equal(dev["k"][mask], k_before[mask]) and torch.equal(dev["v"][mask], v_before[mask])
    o_got = runner.to_f64(call.o)[ids]
    check(f"fp8 layer o (end to end, {len(ids)} sequences)", o_got, ref["o"], t["atol"], t["rel"])
    for i, b in enumerate(ids):
        check(f"fp8 layer o[{b}] (end to end)", o_got[i], ref["o"][i], t["atol"], t["rel"], quiet=True)
    check_lse("fp8 layer lse (end to end)", runner.to_f64(call.lse)[ids], ref["lse"], max(t["lse"], 5e-3))
    check("fp8 layer y (end to end)", runner.to_f64(call.y)[ids], ref["y"], t["atol"], t["rel"])


@pytest.mark.parametrize("G", [0, 3])
def test_layer_fp8_cache_small(G):
    print(f"[case] layer bf16 with e4m3 cache B=5 ctx=300 G={G}", flush=True)
    w = gen.scaled(gen.WORKLOADS["layer_bf16_fp8kv_8k"], batch=5, ctx=300)
    _check_layer_fp8(gen.make_layer(w), num_workgroups=G)


def _layer_workload(cache, w8, batch, ctx):
    # bf16 or block-fp8 weights over a bf16 or e4m3 cache
    if w8:
        kv = gen.BF16 if cache == "bf16" else gen.FP8
        return dataclasses.replace(gen.scaled(gen.WORKLOADS["layer_fp8_8k"], batch=batch, ctx=ctx), kv=kv)
    name = "layer_bf16_8k" if cache == "bf16" else "layer_bf16_fp8kv_8k"
    return gen.scaled(gen.WORKLOADS[name], batch=batch, ctx=ctx)


@pytest.mark.parametrize("w8", [False, True])
@pytest.mark.parametrize("cache", ["bf16", "fp8_e4m3"])
def test_layer_separate_q_and_kv_calls(cache, w8):
    # the layer step with mfa_qproj(_w8) and mfa_kv_append(_fp8/_w8) as two
    # calls (the default step makes them one mfa_qproj_kv_append(_w8) call)
    print(f"[case] layer B=5 ctx=300, {cache} cache, w8={w8}, q path and K/V append as separate calls", flush=True)
    inp = gen.make_layer(_layer_workload(cache, w8, 5, 300))
    if cache == "bf16":
        _check_layer(inp, "bf16", fused=False)
    else:
        _check_layer_fp8(inp, fused=False)


@pytest.mark.parametrize("w8", [False, True])
@pytest.mark.parametrize("cache", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("B", [3, 200])
def test_fused_q_kv_call_matches_the_separate_calls(cache, B, w8):
    # the one-call q path + append against the two calls on the same inputs:
    # q, the appended rows and the lengths agree to fp32 summation order
    # (block-fp8 weights: mfa_qproj_kv_append_w8 against mfa_qproj_w8 +
    # mfa_kv_append_w8)
    print(f"[case] mfa_qproj_kv_append vs mfa_qproj + append, {cache} cache, B={B}, w8={w8}", flush=True)
    inp = gen.make_layer(_layer_workload(cache, w8, B, 40))
    _, dev_f, call_f, _, _ = _run_layer(inp, fused=True)
    runner, dev_s, call_s, _, _ = _run_layer(inp, fused=False)
    assert call_f.fused and not call_s.fused
    assert torch.equal(call_f.len_after, call_s.len_after)
    t = TOL["bf16"]
    check("fused q", runner.to_f64(call_f.q), runner.to_f64(call_s.q), t["atol"], t["rel"])
    rows = torch.as_tensor((inp["seq_off"] + inp["seq_len"]).astype(np.int64), device=dev_f["k"].device)
    if cache == "bf16":
        for nm in ("k", "v"):
            check(f"fused {nm}_new", runner.to_f64(dev_f[nm][rows]), runner.to_f64(dev_s[nm][rows]), t["atol"],
                  t["rel"])
    else:
        tab = om.e4m3fn_table()
        for nm in ("k", "v"):
            a, b = dev_f[nm][rows].cpu().numpy(), dev_s[nm][rows].cpu().numpy()
            # codes may differ by one step where the fp32 value sits at a rounding midpoint
            assert (a == b).mean() >= 0.99, f"{nm}: {(a != b).sum()} codes differ"
            assert np.all(np.abs(tab[a] - tab[b]) <= 0.125 * np.abs(tab[b]) + 2.0 ** -9), nm
    check("fused y", runner.to_f64(call_f.y), runner.to_f64(call_s.y), t["atol"], t["rel"])


def test_layer_fp8_cache_full():
    print("[case] layer layer_bf16_fp8kv_8k (full size, every sequence)", flush=True)
    inp = gen.make_layer(gen.WORKLOADS["layer_bf16_fp8kv_8k"])
    _check_layer_fp8(inp)


# ------------------------------------------------------------------ block-fp8 weights
@pytest.mark.parametrize("kv", [gen.FP8, gen.BF16])
def test_layer_block_fp8_weights_small(kv):
    print(f"[case] layer block-fp8 weights, {kv} cache, B=5 ctx=300", flush=True)
    w = dataclasses.replace(gen.scaled(gen.WORKLOADS["layer_fp8_8k"], batch=5, ctx=300), kv=kv)
    inp = gen.make_layer(w)
    if kv == gen.FP8:
        _check_layer_fp8(inp)
    else:
        _check_layer(inp, "bf16")


def test_layer_block_fp8_weights_batch_200():
    # a second, partly filled 128-row batch chunk in every block-fp8 projection
    print("[case] layer block-fp8 weights, bf16 cache, B=200 ctx=64", flush=True)
    w = dataclasses.replace(gen.scaled(gen.WORKLOADS["layer_fp8_8k"], batch=200, ctx=64), kv=gen.BF16)
    _check_layer(gen.make_layer(w), "bf16")


def test_layer_block_fp8_full():
    print("[case] layer layer_fp8_8k (full size, every sequence)", flush=True)
    inp = gen.make_layer(gen.WORKLOADS["layer_fp8_8k"])
    _check_layer_fp8(inp)


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_kv_append_in_place_length_increment(kv):
    # seq_len_out = seq_len: each row goes to its sequence's old length, then
    # the length advances by one
    from decode_attention_attn_amd import mfa, runner

    print(f"[case] kv append with an in-place length increment, {kv} cache", flush=True)
    wl = "layer_bf16_8k" if kv == "bf16" else "layer_bf16_fp8kv_8k"
    inp = gen.make_layer(gen.scaled(gen.WORKLOADS[wl], batch=6, ctx=50))
    dev = runner.upload_layer(inp)
    B = 6
    ws = torch.empty(mfa.mfa_kv_append_workspace_size(B, mfa.MFA_BF16), dtype=torch.uint8, device="cuda")
    old = dev["len"].clone()
    if kv == "bf16":
        st = mfa.mfa_kv_append(dev["x"], dev["w_k"], dev["w_v"], dev["k"], dev["v"], dev["off"], dev["len"], ws, B,
                               mfa.MFA_BF16, mfa.MFA_BF16, seq_len_out=dev["len"])
    else:
        st = mfa.mfa_kv_append_fp8(dev["x"], dev["w_k"], dev["w_v"], dev["k"], dev["v"], dev["off"], dev["len"],
                                   dev["k_scale"], dev["v_scale"], ws, B, mfa.MFA_BF16, seq_len_out=dev["len"])
    mfa.check(st, "kv append")
    torch.cuda.synchronize()
    assert torch.equal(dev["len"], old + 1)
    ref = om.decode_layer(inp)
    rows = torch.as_tensor((inp["seq_off"] + inp["seq_len"]).astype(np.int64), device=dev["k"].device)
    if kv == "bf16":
        t = TOL["bf16"]
        check("in-place k_new", runner.to_f64(dev["k"][rows]), ref["k_new"], t["atol"], t["rel"])
        check("in-place v_new", runner.to_f64(dev["v"][rows]), ref["v_new"], t["atol"], t["rel"])
    else:
        _check_codes("in-place k codes", dev["k"][rows].cpu().numpy(), ref["k_new_codes"], ref["k_new"],
                     inp["k_scale"])
        _check_codes("in-place v codes", dev["v"][rows].cpu().numpy(), ref["v_new_codes"], ref["v_new"],
                     inp["v_scale"])


def test_kv_append_fp8_f32_activations_and_saturation():
    # fp32 activations (the plain GEMM path) and a scale small enough that
    # part of the row clamps at +-448
    from decode_attention_attn_amd import mfa, runner

    print("[case] kv_append_fp8 f32 activations, saturating scale", flush=True)
    B, cap = 4, 5
    rng = np.random.default_rng(21)
    x = rng.standard_normal((B, 7168)).astype(np.float32)
    w_k = (rng.standard_normal((256, 7168)) / math.sqrt(7168)).astype(np.float32)
    w_v = (rng.standard_normal((256, 7168)) / math.sqrt(7168)).astype(np.float32)
    off = np.arange(B, dtype=np.int64) * cap
    lens = np.array([0, 3, 4, 1], dtype=np.int32)
    kc = rng.integers(0, 0x7F, size=(B * cap, 256), dtype=np.uint8)
    vc = rng.integers(0, 0x7F, size=(B * cap, 256), dtype=np.uint8)
    sk, sv = np.float32(1.0 / 448), np.float32(3.0 / 448)  # |k| > 1 saturates
    d = {n: runner.to_device(a, "f32") for n, a in (("x", x), ("wk", w_k), ("wv", w_v))}
    dk, dv = runner.to_device(kc, "fp8_e4m3"), runner.to_device(vc, "fp8_e4m3")
    doff, dlen = runner.to_device(off, "i64"), runner.to_device(lens, "i32")
    ws = torch.empty(mfa.mfa_kv_append_workspace_size(B, mfa.MFA_F32), dtype=torch.uint8, device="cuda")
    mfa.check(mfa.mfa_kv_append_fp8(d["x"], d["wk"], d["wv"], dk, dv, doff, dlen, sk, sv, ws, B, mfa.MFA_F32),
              "mfa_kv_append_fp8")
    torch.cuda.synchronize()
    k_new, v_new = om.kv_project(x, w_k, w_v)
    assert np.mean(np.abs(k_new / float(sk)) > 448) > 0.2  # the clamp is exercised
    rows = off + lens
    gk, gv = dk.cpu().numpy(), dv.cpu().numpy()
    _check_codes("f32 k_new", gk[rows], om.quantize_e4m3fn(k_new, sk), k_new, sk)
    _check_codes("f32 v_new", gv[rows], om.quantize_e4m3fn(v_new, sv), v_new, sv)
    keep = np.ones(B * cap, dtype=bool)
    keep[rows] = False
    assert np.array_equal(gk[keep], kc[keep]) and np.array_equal(gv[keep], vc[keep])


def _check_replay_against_oracle(runner, dev, call, inp, ref, rep):
    t = TOL["bf16"]
    rows = torch.as_tensor((inp["seq_off"] + inp["seq_len"]).astype(np.int64), device=dev["k"].device)
    check(f"replay {rep} q", runner.to_f64(call.q), ref["q"], t["atol"], t["rel"])
    check(f"replay {rep} k_new", runner.to_f64(dev["k"][rows]), ref["k_new"], t["atol"], t["rel"])
    check(f"replay {rep} v_new", runner.to_f64(dev["v"][rows]), ref["v_new"], t["atol"], t["rel"])
    o = runner.to_f64(call.o)
    check(f"replay {rep} o", o, ref["o"], t["atol"], t["rel"])
    for b in range(len(o)):
        check(f"replay {rep} o[{b}]", o[b], ref["o"][b], t["atol"], t["rel"], quiet=True)
    check_lse(f"replay {rep} lse", runner.to_f64(call.lse), ref["lse"], max(t["lse"], 5e-3))
    check(f"replay {rep} y", runner.to_f64(call.y), ref["y"], t["atol"], t["rel"])


@pytest.mark.parametrize("name,batch,ctx,reps", [("small", 5, 300, 3), ("layer_bf16_8k", None, None, 2)])
def test_layer_step_replays_from_a_hip_graph(name, batch, ctx, reps):
    # The four calls allocate nothing and never wait on the host, so a whole
    # step captures into one HIP graph; every replay (with eager work that
    # clobbers the outputs and restores the cache in between) must equal the
    # eager step bitwise and match the oracle's step on every sequence.
    w = gen.WORKLOADS["layer_bf16_8k"]
    if batch is not None:
        w = gen.scaled(w, batch=batch, ctx=ctx)
    print(f"[case] layer bf16 {name} (B={w.batch}) captured in a HIP graph, {reps} replays", flush=True)
    inp = gen.make_layer(w)
    runner, dev, call, k_before, v_before = _run_layer(inp)
    want = [t.clone() for t in (call.q, call.o, call.lse, call.y, dev["k"], dev["v"])]
    ref = om.decode_layer(inp)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        call()
    torch.cuda.synchronize()
    for rep in range(reps):
        for t in (call.q, call.o, call.lse, call.y):
            t.fill_(float(rep + 7))
        dev["k"].copy_(k_before)
        dev["v"].copy_(v_before)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (call.q, call.o, call.lse, call.y, dev["k"], dev["v"])
        for nm, a, b in zip(("q", "o", "lse", "y", "k", "v"), got, want):
            assert torch.equal(a, b), f"replay {rep}: {nm} differs from the eager step"
        _check_replay_against_oracle(runner, dev, call, inp, ref, rep)
