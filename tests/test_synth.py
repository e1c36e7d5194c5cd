"""The seeded generators: deterministic, the right shapes, valid codes, and a
weight encoding that stays close to the fp32 draw it encodes."""
import numpy as np
import torch

import synth
from oracle import Weights, fused_moe
from oracle import formats as F


def test_generators_are_deterministic_and_shaped():
    wl = synth.WORKLOADS["tiny"]
    a, b = synth.make_weights(wl), synth.make_weights(wl)
    for key in a:
        if a[key] is not None:
            assert torch.equal(a[key], b[key])
    assert a["w13_codes"].shape == (8, 256, 128) and a["w13_scales"].shape == (8, 256, 8)
    assert a["w2_codes"].shape == (8, 256, 64) and a["w2_scales"].shape == (8, 256, 4)
    x = synth.make_x(wl, 16)
    ids, tw = synth.make_routing(wl, 16)
    assert x.dtype == torch.bfloat16 and x.shape == (16, 256)
    assert ids.dtype == torch.int32 and ids.shape == (16, 2)
    assert all(len(set(r)) == 2 for r in ids.tolist())           # distinct experts per token
    assert torch.allclose(tw.sum(1), torch.ones(16))


def test_encodings_track_the_fp32_draw():
    for fmt in ("mxfp4", "nvfp4"):
        w = torch.randn(64, 128, generator=torch.Generator().manual_seed(1)) * 0.02
        if fmt == "mxfp4":
            codes, scales = synth._encode_mxfp4(w)
            dq = F.dequant_mxfp4(codes.numpy(), scales.numpy())
        else:
            codes, scales, g = synth._encode_nvfp4(w)
            assert not np.isnan(F.e4m3_decode(scales.numpy())).any()
            dq = F.dequant_nvfp4(codes.numpy(), scales.numpy(), g.numpy())
        err = np.linalg.norm(dq - w.double().numpy()) / np.linalg.norm(w.double().numpy())
        assert err < 0.2, (fmt, err)


def test_skewed_routing_is_skewed():
    wl = synth.WORKLOADS["skew"]
    ids, _ = synth.make_routing(wl, 2048)
    counts = np.bincount(ids.reshape(-1).numpy(), minlength=wl.E)
    assert counts.max() > 0.6 * 2048 and counts.min() < 64
    assert all(len(set(r)) == wl.k for r in ids[:64].tolist())


def test_oracle_runs_on_tiny_workload():
    wl = synth.WORKLOADS["tiny"]
    wd = synth.oracle_weights_kwargs(synth.make_weights(wl))
    w = Weights(wl.weight_format, wl.gated, **wd)
    x = synth.make_x(wl, 16).view(torch.int16).numpy().view(np.uint16)
    ids, tw = synth.make_routing(wl, 16)
    out = fused_moe(x, ids.numpy(), tw.numpy(), w)
    assert out.shape == (16, 256) and np.isfinite(out).all() and np.abs(out).max() > 0
