"""Dense block-scaled FP4 GEMM (gemm.blockscaled mm) on the GPU against the
fp64 oracle: several tiles of rows with a ragged last tile, a partial N tile,
a ragged last K fragment, one row, a large shape on sampled rows, m = 0, and
the argument checks."""
import numpy as np
import pytest
import torch

import fp8_moe_amd as fm
import synth
from moe_cases import compare
from oracle import blockscaled_mm

pytestmark = pytest.mark.gpu


def dense_problem(m, n, k, fmt, salt=0):
    codes, scales, glob = synth.make_dense_weight(n, k, fmt, seed=salt, device="cuda")
    x = synth.make_dense_x(m, k, seed=salt, device="cuda")
    return codes, scales, glob, x


def oracle_rows(x, codes, scales, glob, fmt, rows=None):
    xs = x if rows is None else x[rows]
    xb = xs.cpu().view(torch.int16).numpy().view(np.uint16)
    g = None if glob is None else np.float32(glob.cpu().item())
    return blockscaled_mm(xb, codes.cpu().numpy(), scales.cpu().numpy(), fmt, g)


CASES = [
    # m, n, k, format, sampled rows
    (1, 256, 2048, "mxfp4", None),
    (7, 4096, 512, "nvfp4", None),
    (300, 512, 1536, "nvfp4", None),       # 3 row tiles, the last ragged
    (129, 48, 96, "mxfp4", None),          # partial N tile, ragged last K fragment
    (130, 272, 160, "nvfp4", None),        # N tile + 16 columns, ragged K
    (4096, 4096, 4096, "nvfp4", [0, 1, 2047, 4000, 4095]),
    (2048, 2048, 7168, "mxfp4", [0, 1023, 2047]),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}_{c[3]}" for c in CASES])
def test_dense_mm_parity(case):
    m, n, k, fmt, rows = case
    print(f"dense mm {case}", flush=True)
    codes, scales, glob, x = dense_problem(m, n, k, fmt)
    wp = fm.gemm_pack_weight(codes, scales, fmt)
    out = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    fm.gemm_mm(x, wp, n, fmt, glob, out=out)
    torch.cuda.synchronize()
    ref = oracle_rows(x, codes, scales, glob, fmt, rows)
    got = out if rows is None else out[rows]
    rel_fro, rel_max, ok = compare(got, ref)
    print(f"  rel_fro={rel_fro:.3e} rel_max={rel_max:.3e}", flush=True)
    assert ok, (rel_fro, rel_max)


def test_dense_mm_strided_rows_and_repeat():
    m, n, k, fmt = 70, 256, 512, "mxfp4"
    codes, scales, glob, x = dense_problem(m, n, k, fmt, salt=1)
    xs = torch.zeros(m, k + 64, dtype=torch.bfloat16, device="cuda")
    xs[:, :k] = x
    out = torch.zeros(m, n + 32, dtype=torch.bfloat16, device="cuda")
    wp = fm.gemm_pack_weight(codes, scales, fmt)
    fm.gemm_mm(xs[:, :k], wp, n, fmt, out=out[:, :n])
    torch.cuda.synchronize()
    first = out.clone()
    fm.gemm_mm(xs[:, :k], wp, n, fmt, out=out[:, :n])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), first.view(torch.int16))  # deterministic
    assert torch.all(out[:, n:] == 0)  # nothing written past n
    rel_fro, rel_max, ok = compare(out[:, :n], oracle_rows(x, codes, scales, glob, fmt))
    assert ok, (rel_fro, rel_max)


def test_dense_mm_zero_rows_and_argument_checks():
    codes, scales, glob, x = dense_problem(4, 64, 128, "nvfp4", salt=2)
    wp = fm.gemm_pack_weight(codes, scales, "nvfp4")
    out = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    fm.gemm_mm(x[:0], wp, 64, "nvfp4", glob, out=out)  # m = 0: no-op
    with pytest.raises(fm.B12xError):
        fm.gemm_mm(x, wp, 64, "nvfp4", None)  # NVFP4 needs the tensor scale
    with pytest.raises(fm.B12xUnsupported):
        fm.gemm_mm(x, wp, 40, "nvfp4", glob)  # n not a multiple of 16
    with pytest.raises(fm.B12xError):
        fm.gemm_mm(x[:, 8:], wp, 64, "nvfp4", glob)  # k = 120: not a multiple of 32
