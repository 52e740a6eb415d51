"""GPU parity of mfa_decode_attn_paged (paged K/V cache) against the float64
oracle (needs an MI355X).

The pages hold the same keys as the packed workloads, in a seeded random page
order, with NaN codes in every row that holds no key (the tail of a
sequence's last page and the spare pages), so a read past a sequence's end or
a wrong page shows as a non-finite or wrong output.
"""

import numpy as np
import pytest

from parity import TOL, check, check_lse

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from decode_attention_attn_amd import inputs as gen  # noqa: E402
from oracle import mfa_oracle as om  # noqa: E402

WL = {"bf16": gen.WORKLOADS["attn_bf16_4k"], "fp8_e4m3": gen.WORKLOADS["attn_fp8kv_4k"]}
LENGTHS = np.array([1, 31, 32, 33, 100, 257, 0, 700, 64, 65], dtype=np.int32)


def _runner():
    from decode_attention_attn_amd import runner  # fails loudly if libmfa.so is missing

    return runner


def _oracle(pg, ids=None):
    return om.decode_attn_paged(pg["q"], pg["k_pages"], pg["v_pages"], pg["block_table"], pg["seq_len"],
                                pg["page_rows"], kind_q=pg["kind_q"], kind_kv=pg["kind_kv"], k_scale=pg["k_scale"],
                                v_scale=pg["v_scale"], batch_ids=ids)


def _run(pg, G=0):
    r = _runner()
    dev = r.upload_attn(pg)
    out, lse = r.AttnCall(dev, G)()
    torch.cuda.synchronize()
    return r.to_f64(out), r.to_f64(lse)


@pytest.mark.parametrize("kind", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("page_rows", [64, 256])
@pytest.mark.parametrize("G", [1, 3, 0])
def test_paged_small(kind, page_rows, G):
    print(f"[case] paged {kind} page_rows={page_rows} G={G} lengths={LENGTHS.tolist()}", flush=True)
    w = gen.scaled(WL[kind], batch=len(LENGTHS), ctx=0, seed=1)
    inp = gen.make_attn(w, lengths=LENGTHS)
    pg = gen.to_pages(inp, page_rows, seed=2)
    out, lse = _run(pg, G)
    o_ref, l_ref = _oracle(pg)
    t = TOL[kind]
    check(f"paged out {kind} R={page_rows} G={G}", out, o_ref, t["atol"], t["rel"])
    check_lse(f"paged lse {kind} R={page_rows} G={G}", lse, l_ref, t["lse"])


@pytest.mark.parametrize("name,page_rows", [
    ("attn_bf16_4k", 64),
    ("attn_fp8kv_4k", 128),
    ("attn_bf16_ragged", 256),
])
def test_paged_full_size(name, page_rows):
    print(f"[case] paged {name} page_rows={page_rows} (full size, every sequence)", flush=True)
    w = gen.WORKLOADS[name]
    inp = gen.make_attn(w)
    pg = gen.to_pages(inp, page_rows, seed=5)
    out, lse = _run(pg)
    o_ref, l_ref = _oracle(pg)
    t = TOL[w.kv]
    check(f"paged {name}", out, o_ref, t["atol"], t["rel"])
    check_lse(f"paged {name} lse", lse, l_ref, t["lse"])
    for b in range(len(out)):
        check(f"paged {name} out[{b}]", out[b], o_ref[b], t["atol"], t["rel"], quiet=True)


def test_paged_matches_contiguous_call():
    # the same keys through both entry points (different work splits, so
    # equal within the bf16 partial rounding, not bitwise)
    print("[case] paged vs contiguous, bf16", flush=True)
    w = gen.scaled(WL["bf16"], batch=6, ctx=0, seed=3)
    inp = gen.make_attn(w, lengths=np.array([3000, 17, 1500, 4096, 0, 129], dtype=np.int32))
    r = _runner()
    o_c, _, _ = r.decode_attn(inp)
    o_p, _ = _run(gen.to_pages(inp, 64, seed=4))
    check("paged vs contiguous", o_p, r.to_f64(o_c), 2e-2, 1e-2)
