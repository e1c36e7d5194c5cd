"""Weight packer on the GPU: the prepared buffer holds exactly the source
codes and scales, byte for byte, at the places the fragment layout assigns
them (layout re-derived here with NumPy reshapes), and zero / neutral scale
padding beyond K."""
import numpy as np
import pytest
import torch

import synth
from moe_cases import small_workload

pytestmark = pytest.mark.gpu


def expected_codes(src, gated):
    """src u8 [E, N, K/2] -> fragments [E, NF, KF, 64 lanes, 16 bytes]."""
    E, N, K2 = src.shape
    K = 2 * K2
    KF = -(-K // 128)
    pad = np.zeros((E, N, KF * 64), np.uint8)
    pad[:, :, :K2] = src
    if gated:   # interleave 16-row blocks: gate block j, up block j
        I = N // 2
        g = pad[:, :I].reshape(E, I // 16, 16, -1)
        u = pad[:, I:].reshape(E, I // 16, 16, -1)
        pad = np.stack([g, u], axis=2).reshape(E, N, -1)
    NF = N // 16
    # [E, NF, 16 rows, KF, 4 groups, 16 bytes] -> [E, NF, KF, group, row, bytes]
    t = pad.reshape(E, NF, 16, KF, 4, 16).transpose(0, 1, 3, 4, 2, 5)
    return t.reshape(E, NF, KF, 64, 16)


def expected_scales(src, gated, nv, KF):
    E, N, nb = src.shape
    per_frag = 8 if nv else 4          # scale codes per fragment row (one per lane group, two for NVFP4)
    fill = 0x38 if nv else 127
    pad = np.full((E, N, KF * per_frag), fill, np.uint8)
    pad[:, :, :nb] = src
    if gated:
        I = N // 2
        g = pad[:, :I].reshape(E, I // 16, 16, -1)
        u = pad[:, I:].reshape(E, I // 16, 16, -1)
        pad = np.stack([g, u], axis=2).reshape(E, N, -1)
    NF = N // 16
    frag_per_word = 2 if nv else 4
    KFS = -(-KF // frag_per_word)
    full = np.full((E, N, KFS * frag_per_word * per_frag), fill, np.uint8)
    full[:, :, :pad.shape[2]] = pad
    if nv:   # [E, NF, 16, KFS, j(2), g(4), h(2)] -> lane (g, row), byte (j, h)
        t = full.reshape(E, NF, 16, KFS, 2, 4, 2).transpose(0, 1, 3, 5, 2, 4, 6)
    else:    # [E, NF, 16, KFS, j(4), g(4)] -> lane (g, row), byte j
        t = full.reshape(E, NF, 16, KFS, 4, 4).transpose(0, 1, 3, 5, 2, 4)
    return t.reshape(E, NF, KFS, 64, 4)


@pytest.mark.parametrize("fmt,gated,H,I", [("mxfp4", True, 256, 128), ("mxfp4", False, 160, 96),
                                           ("nvfp4", True, 160, 96), ("nvfp4", False, 384, 224)])
def test_prepared_layout(fmt, gated, H, I):
    import fp8_moe_amd as fm
    wl = small_workload("pack", 3, H, I, 2, gated, fmt)
    w = synth.make_weights(wl)
    w["w13_codes"] = torch.randint(0, 256, w["w13_codes"].shape, dtype=torch.uint8)   # every nibble value
    wd = {k: (None if v is None else v.cuda()) for k, v in w.items()}
    wp = fm.plan_weights(wl.E, H, I, gated, fmt)
    ex = fm.prepare_weights(wp, wd["w13_codes"], wd["w13_scales"], wd["w2_codes"], wd["w2_scales"],
                            wd["w13_global"], wd["w2_global"])
    torch.cuda.synchronize()
    buf = ex.buffer.cpu().numpy()
    nv = fmt == "nvfp4"
    for name, n, k, gat in (("w13", wl.n13, H, gated), ("w2", H, I, False)):
        codes = expected_codes(w[name + "_codes"].numpy(), gat)
        off = getattr(wp, name + "_codes_off")
        got = buf[off:off + codes.size].reshape(codes.shape)
        assert np.array_equal(got, codes), name
        KF = -(-k // 128)
        sc = expected_scales(w[name + "_scales"].numpy(), gat, nv, KF)
        off = getattr(wp, name + "_scales_off")
        got = buf[off:off + sc.size].reshape(sc.shape)
        assert np.array_equal(got, sc), name
    if nv:
        for name in ("w13", "w2"):
            off = getattr(wp, name + "_global_off")
            assert np.array_equal(buf[off:off + 4 * wl.E].view(np.float32), w[name + "_global"].numpy())
