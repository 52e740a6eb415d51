"""GPU parity of the projection calls at batch sizes around the GEMM planner's
choices, against the float64 oracle (needs an MI355X).

bf16 weights take 64-column tiles while a product's activations fit in L2
(batch x K x 2 bytes <= 2 MB) and 128-column tiles with a nontemporal weight
stream above that; the split-K count follows the tile count; a batch above 128
rows adds batch chunks, the last one partly filled. The cases below cross each
of those boundaries for the out-projection (K = 16384: 64 rows and fewer vs 65
and more), the q path (q down K = 7168: 146 rows; q up K = 2048: 512 rows) and
the stacked [W_dq; W_k; W_v] product of mfa_qproj_kv_append. Rows are checked
on a sample (every output row is computed independently, so the oracle only
runs those rows).
"""

import numpy as np
import pytest

from parity import TOL, check

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from decode_attention_attn_amd import inputs as gen  # noqa: E402
from oracle import mfa_oracle as om  # noqa: E402


def _rows(B):
    """A sample of batch rows: the first and last of every 128-row chunk and a few inside."""
    rows = set()
    for c0 in range(0, B, 128):
        c1 = min(B, c0 + 128)
        rows.update(range(c0, min(c1, c0 + 4)))
        rows.update(range(max(c0, c1 - 4), c1))
        rows.add((c0 + c1) // 2)
    return sorted(rows)


def _bf16(seed, tid, shape, scale=None):
    return gen.store(gen.normal(seed, tid, shape, scale), gen.BF16)


@pytest.mark.parametrize("B", [1, 64, 65, 130])
def test_oproj_across_tile_choices(B):
    from decode_attention_attn_amd import mfa, runner

    print(f"[case] mfa_oproj bf16 B={B}", flush=True)
    o = _bf16(21, 1, (B, 16384))
    w = gen.store(gen.weight(21, 2, 7168, 16384), gen.BF16)
    y = torch.empty((B, 7168), dtype=torch.bfloat16, device="cuda")
    ws = runner._ws(mfa.mfa_oproj_workspace_size(B, mfa.MFA_BF16), "cuda")
    mfa.check(mfa.mfa_oproj(runner.to_device(o, gen.BF16), runner.to_device(w, gen.BF16), y, ws, B, mfa.MFA_BF16),
              "mfa_oproj")
    torch.cuda.synchronize()
    rows = _rows(B)
    ref = om.out_proj(om.to_f64(o[rows], gen.BF16), om.to_f64(w, gen.BF16))
    t = TOL["bf16"]
    check(f"oproj y B={B}", runner.to_f64(y)[rows], ref, t["atol"], t["rel"])


@pytest.mark.parametrize("B", [1, 150, 520])
def test_qproj_across_tile_choices(B):
    from decode_attention_attn_amd import mfa, runner

    print(f"[case] mfa_qproj bf16 B={B}", flush=True)
    x = _bf16(22, 1, (B, 7168))
    w_dq = gen.store(gen.weight(22, 2, 2048, 7168), gen.BF16)
    w_uq = gen.store(gen.weight(22, 3, 16384, 2048), gen.BF16)
    q = torch.empty((B, 64, 256), dtype=torch.bfloat16, device="cuda")
    ws = runner._ws(mfa.mfa_qproj_workspace_size(B, mfa.MFA_BF16), "cuda")
    mfa.check(mfa.mfa_qproj(runner.to_device(x, gen.BF16), runner.to_device(w_dq, gen.BF16), None, 1e-6,
                            runner.to_device(w_uq, gen.BF16), q, ws, B, mfa.MFA_BF16), "mfa_qproj")
    torch.cuda.synchronize()
    rows = _rows(B)
    _, _, ref = om.q_path(om.to_f64(x[rows], gen.BF16), om.to_f64(w_dq, gen.BF16), om.to_f64(w_uq, gen.BF16))
    t = TOL["bf16"]
    check(f"qproj q B={B}", runner.to_f64(q)[rows], ref, t["atol"], t["rel"])


@pytest.mark.parametrize("B", [150])
def test_qproj_kv_append_wide_tiles(B):
    # 150 rows of 7168: 2.1 MB of activations, so the stacked product takes
    # 128-column tiles (the layer tests at 128 and 200 rows cover 64 and 128)
    from decode_attention_attn_amd import mfa, runner

    print(f"[case] mfa_qproj_kv_append bf16 B={B}", flush=True)
    ctx = 16
    x = _bf16(23, 1, (B, 7168))
    w_dq = gen.store(gen.weight(23, 2, 2048, 7168), gen.BF16)
    w_uq = gen.store(gen.weight(23, 3, 16384, 2048), gen.BF16)
    w_k = gen.store(gen.weight(23, 4, 256, 7168), gen.BF16)
    w_v = gen.store(gen.weight(23, 5, 256, 7168), gen.BF16)
    cap = ctx + 1
    k_cache = torch.zeros((B * cap, 256), dtype=torch.bfloat16, device="cuda")
    v_cache = torch.zeros((B * cap, 256), dtype=torch.bfloat16, device="cuda")
    seq_off = torch.arange(B, dtype=torch.int64, device="cuda") * cap
    seq_len = torch.full((B,), ctx, dtype=torch.int32, device="cuda")
    q = torch.empty((B, 64, 256), dtype=torch.bfloat16, device="cuda")
    ws = runner._ws(mfa.mfa_qproj_kv_append_workspace_size(B), "cuda")
    dv = lambda a: runner.to_device(a, gen.BF16)  # noqa: E731
    mfa.check(mfa.mfa_qproj_kv_append(dv(x), dv(w_dq), None, 1e-6, dv(w_uq), dv(w_k), dv(w_v), q, k_cache, v_cache,
                                      seq_off, seq_len, 1.0, 1.0, ws, B, mfa.MFA_BF16), "mfa_qproj_kv_append")
    torch.cuda.synchronize()
    rows = _rows(B)
    xr = om.to_f64(x[rows], gen.BF16)
    _, _, q_ref = om.q_path(xr, om.to_f64(w_dq, gen.BF16), om.to_f64(w_uq, gen.BF16))
    k_ref, v_ref = om.kv_project(xr, om.to_f64(w_k, gen.BF16), om.to_f64(w_v, gen.BF16))
    t = TOL["bf16"]
    check(f"qkv q B={B}", runner.to_f64(q)[rows], q_ref, t["atol"], t["rel"])
    at = torch.as_tensor([r * cap + ctx for r in rows], device="cuda")
    check(f"qkv k_new B={B}", runner.to_f64(k_cache[at]), k_ref, t["atol"], t["rel"])
    check(f"qkv v_new B={B}", runner.to_f64(v_cache[at]), v_ref, t["atol"], t["rel"])
    # no other cache row was written
    mask = torch.ones(B * cap, dtype=torch.bool, device="cuda")
    mask[seq_off + ctx] = False
    assert not k_cache[mask].any() and not v_cache[mask].any()
