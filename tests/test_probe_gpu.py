"""GPU check of mfa_bw_probe, the streaming-read bandwidth probe that the
benchmark compares the KV rate with (needs an MI355X): the XOR of the
per-workgroup checksums equals the XOR of every 32-bit word of the buffer,
bit for bit, for sizes with ragged tails and several workgroup counts."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (3 << 20) + 48, 64 << 20])
@pytest.mark.parametrize("G", [1, 7, 0])
def test_probe_checksum_is_exact(nbytes, G):
    from decode_attention_attn_amd import mfa

    print(f"[case] bw probe {nbytes} bytes, G={G}", flush=True)
    words = np.random.default_rng([nbytes, G]).integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n_sink = G if G > 0 else cus
    sink = torch.full((n_sink,), -1, dtype=torch.int32, device="cuda")
    mfa.check(mfa.mfa_bw_probe(buf, sink, G), "mfa_bw_probe")
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(words)
    assert int(got) == int(want), (hex(int(got)), hex(int(want)))
