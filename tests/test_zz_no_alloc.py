"""mfa_decode_attn_noalloc (no workspace argument: the library's static
per-GPU scratch) against mfa_decode_attn with a caller's workspace (needs an
MI355X).

The two run the same kernels with the same work split, so their outputs must
agree bit for bit; each is also held to the oracle. Two calls follow each
other on the shared buffer, the second with a smaller batch, so whatever the
first left there must not leak into the second. A batch whose workspace would
exceed the buffer is rejected on the host.
"""

import numpy as np
import pytest

from parity import TOL, check, check_lse

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from decode_attention_attn_amd import inputs as gen  # noqa: E402
from oracle import mfa_oracle as om  # noqa: E402

WL = {
    "bf16": gen.WORKLOADS["attn_bf16_4k"],
    "fp8_e4m3": gen.WORKLOADS["attn_fp8kv_4k"],
    "f32": gen.Workload("attn_f32", "attn", 8, 0, gen.F32, gen.F32),
}
FIRST = np.array([3000, 17, 1500, 4096, 0, 129, 777, 2048], dtype=np.int32)
SECOND = np.array([65, 1, 300], dtype=np.int32)


def _make(kind, lengths, seed):
    w = gen.scaled(WL[kind], batch=len(lengths), ctx=0, seed=seed)
    return gen.make_attn(w, lengths=lengths)


def _noalloc(runner, dev, G):
    from decode_attention_attn_amd import mfa

    out = torch.empty((dev["B"], 64, 256), dtype=torch.float32 if dev["kind_q"] == gen.F32 else torch.bfloat16,
                      device=dev["q"].device)
    lse = torch.empty((dev["B"], 64), dtype=torch.float32, device=dev["q"].device)
    st = mfa.mfa_decode_attn_noalloc(dev["q"], dev["k"], dev["v"], dev["off"], dev["len"], runner.SOFTMAX_SCALE,
                                     dev["k_scale"], dev["v_scale"], out, lse, dev["B"], G,
                                     runner.dtype_code(dev["kind_q"]), runner.dtype_code(dev["kind_kv"]))
    mfa.check(st, "mfa_decode_attn_noalloc")
    return out, lse


@pytest.mark.parametrize("kind", ["bf16", "fp8_e4m3", "f32"])
@pytest.mark.parametrize("G", [0, 3])
def test_noalloc_equals_workspace_call_on_two_calls(kind, G):
    from decode_attention_attn_amd import runner

    for step, (lengths, seed) in enumerate(((FIRST, 11), (SECOND, 12))):
        print(f"[case] noalloc {kind} G={G} call {step} lengths={lengths.tolist()}", flush=True)
        inp = _make(kind, lengths, seed)
        dev = runner.upload_attn(inp)
        o_ws, l_ws = runner.AttnCall(dev, G)()
        o_na, l_na = _noalloc(runner, dev, G)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ws), f"call {step}: output differs from the workspace call"
        assert torch.equal(l_na, l_ws), f"call {step}: lse differs from the workspace call"
        o_ref, l_ref = om.decode_attn(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_off"], inp["seq_len"],
                                      kind_q=inp["kind_q"], kind_kv=inp["kind_kv"], k_scale=inp["k_scale"],
                                      v_scale=inp["v_scale"])
        t = TOL[kind]
        check(f"noalloc out {kind} G={G} call {step}", runner.to_f64(o_na), o_ref, t["atol"], t["rel"])
        check_lse(f"noalloc lse {kind} G={G} call {step}", runner.to_f64(l_na), l_ref, t["lse"])


def test_noalloc_rejects_a_batch_beyond_its_buffer():
    from decode_attention_attn_amd import mfa

    G = 256
    B = 1000
    assert mfa.mfa_decode_attn_workspace_size(B, G) > mfa.MFA_NOALLOC_SCRATCH_BYTES
    assert mfa.mfa_decode_attn_workspace_size(300, G) <= mfa.MFA_NOALLOC_SCRATCH_BYTES
    fake = 0x10000  # never dereferenced: the size check fails before any launch
    st = mfa.raw_function("mfa_decode_attn_noalloc")(fake, fake, fake, fake, fake, 0.0625, 1.0, 1.0, fake, None, B, G,
                                                    mfa.MFA_BF16, mfa.MFA_BF16, None)
    assert st == mfa.MFA_ERR_WORKSPACE
