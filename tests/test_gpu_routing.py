"""Routing stage on the GPU: counts, offsets, padded offsets, the stable
permutation and pair positions bit-exact with the oracle; the tile list
(one of many valid ones) checked for validity by the oracle's checker."""
import numpy as np
import pytest
import torch

import synth
from moe_cases import small_workload
from oracle.routing import check_tiles, route

pytestmark = pytest.mark.gpu


def _ids(kind, T, k, E, seed):
    g = torch.Generator().manual_seed(seed)
    if kind == "uniform":
        return torch.topk(torch.rand(T, E, generator=g), k, dim=1).indices.to(torch.int32)
    if kind == "one_expert":
        return torch.full((T, k), E - 1, dtype=torch.int32)
    if kind == "duplicates":
        return torch.randint(0, 3, (T, k), generator=g, dtype=torch.int32)
    if kind == "bad_ids":
        ids = torch.randint(-3, E + 3, (T, k), generator=g, dtype=torch.int32)
        ids[0, 0] = -(2 ** 31)
        ids[-1, -1] = 2 ** 31 - 1
        return ids
    if kind == "zipf":
        wl = synth.Workload("z", E, 32, 32, k, True, "mxfp4", "bf16", (T,), "zipf")
        return synth.make_routing(wl, T)[0]
    raise ValueError(kind)


CASES = [
    ("uniform", 16, 2, 8), ("uniform", 1, 8, 128), ("uniform", 4096, 8, 128), ("uniform", 1000, 3, 64),
    ("one_expert", 700, 4, 16), ("duplicates", 333, 5, 8), ("bad_ids", 513, 4, 32), ("zipf", 2048, 8, 256),
    ("uniform", 37, 1, 1), ("uniform", 300, 4, 1024),
]


@pytest.mark.parametrize("kind,T,k,E", CASES)
def test_routing_bit_exact(kind, T, k, E):
    import fp8_moe_amd as fm
    print(f"routing case {kind} T={T} k={k} E={E}", flush=True)
    ids = _ids(kind, T, k, E, seed=T * 31 + k)
    wl = small_workload("route", E, 32, 32, k)
    wd = {key: torch.zeros(E, *shape, dtype=torch.uint8, device="cuda") for key, shape in
          (("w13_codes", (64, 16)), ("w13_scales", (64, 1)), ("w2_codes", (32, 16)), ("w2_scales", (32, 1)))}
    model = fm.FusedMoE(E, 32, 32, k, "mxfp4", "bf16", "silu", T, wd, decode_max_pairs=-1)
    x = torch.zeros(T, 32, dtype=torch.bfloat16, device="cuda")
    tw = torch.ones(T, k, dtype=torch.float32, device="cuda")
    b, out = model.bind(x, ids.cuda(), tw)
    fm.run_stage(b, "route")
    torch.cuda.synchronize()
    ref = route(ids.numpy(), E, fm.binding_query(b, "row_pad"), fm.binding_query(b, "tile_rows"))

    def region(name, count):
        off, nbytes = model.plan.scratch_region(name)
        assert count * 4 <= nbytes
        return model.scratch[off:off + 4 * count].cpu().numpy().view(np.int32)

    assert np.array_equal(region("counts", E), ref.counts)
    assert np.array_equal(region("offsets", E + 1), ref.offsets)
    assert np.array_equal(region("padded_offsets", E + 1), ref.padded_offsets)
    nt = region("ntiles", 4)
    assert nt[1] == ref.padded_offsets[-1]
    assert np.array_equal(region("sorted", int(ref.padded_offsets[-1])), ref.sorted_ids)
    assert np.array_equal(region("pos", T * k), ref.pos)
    off, nbytes = model.plan.scratch_region("tiles")
    assert 0 <= nt[0] <= nbytes // 16
    tiles = region("tiles", 4 * int(nt[0])).reshape(-1, 4)
    problems = check_tiles(tiles[:, :3], nt[0], ref.padded_offsets, E, fm.binding_query(b, "row_pad"),
                           fm.binding_query(b, "tile_rows"))
    assert problems == [], problems[:5]
