"""The benchmark harness's measurement probes (libb12x_probes.so) read what
they claim to read and run the MFMAs they claim to run: the stream-read digest
equals the XOR of each thread's words computed on the host, and the MFMA
probe's result is linear in the number of rounds and the same for bf16 and f16
operands (its operands are exact in both)."""
import numpy as np
import pytest
import torch

from bench import ProbeError, probe_mfma, probe_stream_read

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("workgroups,words_per_wg", [(4, 2048), (3, 1024 + 517), (1, 700)])
def test_stream_read_digest(workgroups, words_per_wg):
    g = torch.Generator().manual_seed(workgroups * 1000 + words_per_wg)
    total = workgroups * words_per_wg + 5  # a few words past the last share
    host = torch.randint(-2**31, 2**31 - 1, (total * 4,), dtype=torch.int64, generator=g).to(torch.int32)
    src = host.cuda()
    sink = torch.zeros(workgroups * 256, dtype=torch.int32, device="cuda")
    probe_stream_read(src, sink, workgroups)
    torch.cuda.synchronize()
    words = host.numpy().view(np.uint32).reshape(total, 4)
    per = total // workgroups
    chunks = per // 1024
    want = np.zeros((workgroups, 256), np.uint32)
    for b in range(workgroups):
        share = words[b * per: b * per + chunks * 1024].reshape(chunks * 4, 256, 4)
        want[b] = np.bitwise_xor.reduce(np.bitwise_xor.reduce(share, axis=2), axis=0) if chunks else 0
    got = sink.cpu().numpy().view(np.uint32).reshape(workgroups, 256)
    np.testing.assert_array_equal(got, want)


def test_mfma_probe_linear_and_dtype_independent():
    wg = 8
    out = {}
    for f16 in (False, True):
        for it in (1, 3):
            sink = torch.full((wg * 256,), float("nan"), dtype=torch.float32, device="cuda")
            probe_mfma(sink, wg, it, f16=f16)
            torch.cuda.synchronize()
            out[f16, it] = sink.cpu()
    one = out[False, 1]
    assert torch.isfinite(one).all() and (one > 0).all()
    torch.testing.assert_close(out[False, 3], 3 * one, rtol=0, atol=0)
    torch.testing.assert_close(out[True, 1], one, rtol=0, atol=0)
    torch.testing.assert_close(out[True, 3], 3 * one, rtol=0, atol=0)
    # every workgroup computes the same thing
    per_wg = one.view(wg, 256)
    assert (per_wg == per_wg[0]).all()


def test_probe_errors():
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    src = torch.zeros(64, dtype=torch.int32, device="cuda")
    with pytest.raises(ProbeError):
        probe_stream_read(src, sink, 0)
    with pytest.raises(ProbeError):
        probe_stream_read(src[1:], sink, 1)  # 4-byte offset: misaligned, and not a multiple of 16
    with pytest.raises(ProbeError):
        probe_mfma(torch.zeros(256, device="cuda"), 1, 0)
