"""GPU parity of the whole decode step (mfa_qproj, mfa_kv_append,
mfa_decode_attn, mfa_oproj) against the float64 oracle (needs an MI355X).

Checked per stage: q, the appended K/V rows (and that no other cache byte
changed), the attention output and lse, and y. "End to end" compares with the
oracle run from the stored inputs alone; "stage isolated" feeds the oracle's
attention the GPU's own q and cache, so each kernel's error is seen alone.
"""

import numpy as np
import pytest

from parity import TOL, check, check_lse

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from decode_attention_attn_amd import inputs as gen  # noqa: E402
from oracle import mfa_oracle as om  # noqa: E402


def _run_layer(inp, num_workgroups=0):
    from decode_attention_attn_amd import runner

    dev = runner.upload_layer(inp)
    k_before = dev["k"].clone()
    v_before = dev["v"].clone()
    call = runner.LayerCall(dev, num_workgroups)
    call()
    torch.cuda.synchronize()
    return runner, dev, call, k_before, v_before


def _check_layer(inp, ids, kind, num_workgroups=0):
    runner, dev, call, k_before, v_before = _run_layer(inp, num_workgroups)
    t = TOL[kind]
    ref = om.decode_layer(inp, batch_ids=ids)
    B = len(inp["seq_len"])
    rows = (inp["seq_off"] + inp["seq_len"]).astype(np.int64)
    # q and the appended rows, for every sequence
    ref_all = om.decode_layer(inp, batch_ids=list(range(B))) if B <= 8 else None
    if ref_all is not None:
        q_ref, k_ref, v_ref = ref_all["q"], ref_all["k_new"], ref_all["v_new"]
        q_ids = list(range(B))
    else:
        q_ref, k_ref, v_ref, q_ids = ref["q"], ref["k_new"], ref["v_new"], ids
    check(f"{kind} q", runner.to_f64(call.q)[q_ids], q_ref, t["atol"], t["rel"])
    k_new = runner.to_f64(dev["k"][torch.as_tensor(rows[q_ids], device=dev["k"].device)])
    v_new = runner.to_f64(dev["v"][torch.as_tensor(rows[q_ids], device=dev["v"].device)])
    check(f"{kind} k_new", k_new, k_ref, t["atol"], t["rel"])
    check(f"{kind} v_new", v_new, v_ref, t["atol"], t["rel"])
    # no other cache row changed
    mask = torch.ones(dev["k"].shape[0], dtype=torch.bool, device=dev["k"].device)
    mask[torch.as_tensor(rows, device=mask.device)] = False
    assert torch.equal(dev["k"][mask], k_before[mask]) and torch.equal(dev["v"][mask], v_before[mask])
    # attention and output, end to end
    check(f"{kind} o (end to end)", runner.to_f64(call.o)[ids], ref["o"], t["atol"], t["rel"])
    check_lse(f"{kind} lse (end to end)", runner.to_f64(call.lse)[ids], ref["lse"], max(t["lse"], 5e-3))
    check(f"{kind} y (end to end)", runner.to_f64(call.y)[ids], ref["y"], t["atol"], t["rel"])
    # stage isolated: oracle attention on the GPU's q and cache, oracle y on the GPU's o
    qg = runner.to_f64(call.q)[ids]
    lens = inp["seq_len"][ids] + 1
    spans = [torch.arange(int(inp["seq_off"][b]), int(inp["seq_off"][b]) + int(n), device=dev["k"].device)
             for b, n in zip(ids, lens)]
    sel = torch.cat(spans)
    kc, vc = runner.to_f64(dev["k"][sel]), runner.to_f64(dev["v"][sel])
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    o_iso, l_iso = om.decode_attn(qg, kc, vc, offs, lens)
    check(f"{kind} o (stage isolated)", runner.to_f64(call.o)[ids], o_iso, t["atol"], t["rel"])
    y_iso = om.out_proj(runner.to_f64(call.o)[ids], om.to_f64(inp["w_o"], inp["kind_act"]))
    check(f"{kind} y (stage isolated)", runner.to_f64(call.y)[ids], y_iso, t["atol"], t["rel"])


def test_layer_tiny_fp32_full():
    print("[case] layer tiny_fp32 (full size)", flush=True)
    inp = gen.make_layer(gen.WORKLOADS["tiny_fp32"])
    _check_layer(inp, [0, 1], "f32")


@pytest.mark.parametrize("G", [0, 3])
def test_layer_bf16_small(G):
    print(f"[case] layer bf16 small B=5 ctx=300 G={G}", flush=True)
    w = gen.scaled(gen.WORKLOADS["layer_bf16_8k"], batch=5, ctx=300)
    inp = gen.make_layer(w)
    _check_layer(inp, [0, 2, 4], "bf16", num_workgroups=G)


@pytest.mark.parametrize("B", [1, 200])
def test_layer_bf16_batch_edges(B):
    # one sequence; and more sequences than one 128-row GEMM tile (a second,
    # partly filled batch chunk in every projection)
    print(f"[case] layer bf16 B={B} ctx=64", flush=True)
    w = gen.scaled(gen.WORKLOADS["layer_bf16_8k"], batch=B, ctx=64)
    inp = gen.make_layer(w)
    ids = [0] if B == 1 else [0, 127, 128, 199]
    _check_layer(inp, ids, "bf16")


def test_layer_bf16_8k_full():
    print("[case] layer layer_bf16_8k (full size, sampled sequences)", flush=True)
    inp = gen.make_layer(gen.WORKLOADS["layer_bf16_8k"])
    _check_layer(inp, [0, 77, 127], "bf16")
