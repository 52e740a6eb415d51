"""GPU parity of mfa_decode_attn_mt and mfa_decode_attn_paged_mt (2 to 4 new
query tokens per sequence, causal among them) against the float64 oracle
(needs an MI355X)."""

import numpy as np
import pytest

from parity import TOL, check, check_lse

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from decode_attention_attn_amd import inputs as gen  # noqa: E402
from oracle import mfa_oracle as om  # noqa: E402

WL = {"bf16": gen.WORKLOADS["attn_bf16_4k"], "fp8_e4m3": gen.WORKLOADS["attn_fp8kv_4k"]}
# lengths below n_tokens: the first tokens see no row (output 0, lse -inf);
# 0: empty sequence
LENGTHS = np.array([2, 1, 31, 32, 33, 100, 257, 0, 700, 65, 3, 4], dtype=np.int32)


def _run(inp, G=0):
    from decode_attention_attn_amd import runner

    dev = runner.upload_attn(inp)
    out, lse = runner.AttnCall(dev, G)()
    torch.cuda.synchronize()
    return runner, runner.to_f64(out), runner.to_f64(lse)


def _oracle(inp, ids=None):
    return om.decode_attn_mt(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_off"], inp["seq_len"],
                             inp["n_tokens"], kind_q=inp["kind_q"], kind_kv=inp["kind_kv"], k_scale=inp["k_scale"],
                             v_scale=inp["v_scale"], batch_ids=ids)


@pytest.mark.parametrize("nt", [2, 3, 4])
@pytest.mark.parametrize("kind", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("G", [1, 3, 0])
def test_tokens_small(nt, kind, G):
    print(f"[case] {nt} tokens {kind} G={G} lengths={LENGTHS.tolist()}", flush=True)
    w = gen.scaled(WL[kind], batch=len(LENGTHS), ctx=0, seed=2)
    inp = gen.with_tokens(gen.make_attn(w, lengths=LENGTHS), nt)
    _, out, lse = _run(inp, G)
    o_ref, l_ref = _oracle(inp)
    t = TOL[kind]
    check(f"{nt} tokens out {kind} G={G}", out, o_ref, t["atol"], t["rel"])
    check_lse(f"{nt} tokens lse {kind} G={G}", lse, l_ref, t["lse"])


def _oracle_paged(pg, ids=None):
    return om.decode_attn_paged_mt(pg["q"], pg["k_pages"], pg["v_pages"], pg["block_table"], pg["seq_len"],
                                   pg["page_rows"], pg["n_tokens"], kind_q=pg["kind_q"], kind_kv=pg["kind_kv"],
                                   k_scale=pg["k_scale"], v_scale=pg["v_scale"], batch_ids=ids)


@pytest.mark.parametrize("nt", [2, 3, 4])
@pytest.mark.parametrize("kind", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("page_rows,G", [(64, 1), (64, 0), (256, 3)])
def test_tokens_paged_small(nt, kind, page_rows, G):
    # several tokens over shuffled pages whose unused rows hold NaN codes
    print(f"[case] {nt} tokens paged {kind} page_rows={page_rows} G={G} lengths={LENGTHS.tolist()}", flush=True)
    w = gen.scaled(WL[kind], batch=len(LENGTHS), ctx=0, seed=4)
    pg = gen.to_pages(gen.with_tokens(gen.make_attn(w, lengths=LENGTHS), nt), page_rows, seed=6)
    _, out, lse = _run(pg, G)
    o_ref, l_ref = _oracle_paged(pg)
    t = TOL[kind]
    check(f"{nt} tokens paged out {kind} R={page_rows} G={G}", out, o_ref, t["atol"], t["rel"])
    check_lse(f"{nt} tokens paged lse {kind} R={page_rows} G={G}", lse, l_ref, t["lse"])


@pytest.mark.parametrize("name,page_rows,nt", [("attn_bf16_4k", 64, 2), ("attn_fp8kv_4k", 128, 2),
                                               ("attn_bf16_4k", 128, 3)])
def test_tokens_paged_full_size(name, page_rows, nt):
    print(f"[case] {nt} tokens paged {name} page_rows={page_rows} (full size, every sequence)", flush=True)
    w = gen.WORKLOADS[name]
    pg = gen.to_pages(gen.with_tokens(gen.make_attn(w), nt), page_rows, seed=7)
    _, out, lse = _run(pg)
    o_ref, l_ref = _oracle_paged(pg)
    t = TOL[w.kv]
    check(f"{nt} tokens paged {name}", out, o_ref, t["atol"], t["rel"])
    check_lse(f"{nt} tokens paged {name} lse", lse, l_ref, t["lse"])
    for b in range(len(out)):
        check(f"{nt} tokens paged {name} out[{b}]", out[b], o_ref[b], t["atol"], t["rel"], quiet=True)


@pytest.mark.parametrize("name,nt", [("attn_bf16_4k", 2), ("attn_fp8kv_4k", 2), ("attn_bf16_4k", 4),
                                     ("attn_fp8kv_4k", 4)])
def test_tokens_full_size(name, nt):
    print(f"[case] {nt} tokens {name} (full size, every sequence)", flush=True)
    w = gen.WORKLOADS[name]
    inp = gen.with_tokens(gen.make_attn(w), nt)
    _, out, lse = _run(inp)
    o_ref, l_ref = _oracle(inp)
    t = TOL[w.kv]
    check(f"{nt} tokens {name}", out, o_ref, t["atol"], t["rel"])
    check_lse(f"{nt} tokens {name} lse", lse, l_ref, t["lse"])
    for b in range(len(out)):
        check(f"{nt} tokens {name} out[{b}]", out[b], o_ref[b], t["atol"], t["rel"], quiet=True)


def test_one_token_through_the_multi_token_entry_is_the_single_token_call():
    print("[case] n_tokens = 1 via mfa_decode_attn_mt vs mfa_decode_attn", flush=True)
    from decode_attention_attn_amd import mfa, runner

    w = gen.scaled(WL["bf16"], batch=6, ctx=0, seed=3)
    inp = gen.make_attn(w, lengths=np.array([3000, 17, 1500, 4096, 0, 129], dtype=np.int32))
    o1, l1, dev = runner.decode_attn(inp)
    B = dev["B"]
    out = torch.empty_like(o1)
    lse = torch.empty_like(l1)
    ws = torch.empty(mfa.mfa_decode_attn_mt_workspace_size(B, 1, 0), dtype=torch.uint8, device="cuda")
    mfa.check(mfa.mfa_decode_attn_mt(dev["q"], dev["k"], dev["v"], dev["off"], dev["len"], 1, 0.0625, 1.0, 1.0, out,
                                     lse, ws, B, 0, mfa.MFA_BF16, mfa.MFA_BF16), "mfa_decode_attn_mt")
    torch.cuda.synchronize()
    assert torch.equal(out, o1) and torch.equal(lse, l1)


@pytest.mark.parametrize("kind", ["bf16", "fp8_e4m3"])
def test_one_token_through_the_paged_multi_token_entry_is_the_paged_call(kind):
    print(f"[case] n_tokens = 1 via mfa_decode_attn_paged_mt vs mfa_decode_attn_paged, {kind}", flush=True)
    from decode_attention_attn_amd import mfa, runner

    w = gen.scaled(WL[kind], batch=6, ctx=0, seed=8)
    pg = gen.to_pages(gen.make_attn(w, lengths=np.array([3000, 17, 1500, 4096, 0, 129], dtype=np.int32)), 64,
                      seed=9)
    dev = runner.upload_attn(pg)
    o1, l1 = runner.AttnCall(dev)()
    B = dev["B"]
    out = torch.empty_like(o1)
    lse = torch.empty_like(l1)
    ws = torch.empty(mfa.mfa_decode_attn_mt_workspace_size(B, 1, 0), dtype=torch.uint8, device="cuda")
    mfa.check(mfa.mfa_decode_attn_paged_mt(dev["q"], dev["k"], dev["v"], dev["table"], dev["max_blocks"],
                                           dev["page_rows"], dev["len"], 1, 0.0625, dev["k_scale"], dev["v_scale"],
                                           out, lse, ws, B, 0, mfa.MFA_BF16, runner.dtype_code(kind)),
              "mfa_decode_attn_paged_mt")
    torch.cuda.synchronize()
    assert torch.equal(out, o1) and torch.equal(lse, l1)
