"""kvs_gather_read_floor (a measurement kernel, not a step of the method) through the C ABI (needs an
MI355X): every listed tile's K and V values are read and summed, checked against a float64 sum of the
same tiles, with and without reserved LDS."""
from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("no GPU", allow_module_level=True)

from block_sparse_kv_amd import binding as Bd  # noqa: E402

import kvsynth  # noqa: E402

DEV = "cuda"
B = D = 128


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("lds", [0, 36864])
def test_gather_read_floor_sums(lds):
    n_phys, Hkv = 13, 4
    say(f"[case] gather read floor: {n_phys} blocks x {Hkv} KV heads, lds {lds}")
    kp = kvsynth.randn_fp16((n_phys, Hkv, B, D), 71, DEV)
    vp = kvsynth.randn_fp16((n_phys, Hkv, B, D), 72, DEV)
    rng = np.random.default_rng(5)
    ids = rng.integers(0, n_phys * Hkv, size=37).astype(np.int32)
    ids[:3] = [0, n_phys * Hkv - 1, 0]  # first and last tile, and a repeat
    ids[3:5] = [n_phys * Hkv, -1]       # outside the pools: nothing read, NaN
    tid = torch.from_numpy(ids).to(DEV)
    out = torch.full((len(ids),), float("nan"), dtype=torch.float32, device=DEV)
    Bd.kvs_gather_read_floor(kp, vp, n_phys * Hkv, tid, len(ids), lds, out)
    torch.cuda.synchronize()
    kt = kp.view(-1, B * D).double().cpu().numpy()
    vt = vp.view(-1, B * D).double().cpu().numpy()
    got = out.double().cpu().numpy()
    assert np.isnan(got[3]) and np.isnan(got[4])
    ok = np.r_[0:3, 5:len(ids)]
    ref = kt[ids[ok]].sum(axis=1) + vt[ids[ok]].sum(axis=1)
    mag = np.abs(kt[ids[ok]]).sum(axis=1) + np.abs(vt[ids[ok]]).sum(axis=1)
    err = np.abs(got[ok] - ref)
    assert np.all(err <= 2e-5 * mag + 1e-3), (err.max(), mag.min())
    assert Bd.kvs_gather_read_floor(kp, vp, n_phys * Hkv, tid, 0, lds, out, check=False) == Bd.KVS_OK
    say(f"[ok] gather read floor: max err {err.max():.2e} over {len(ids)} tiles")
