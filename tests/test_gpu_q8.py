"""The Q8_0, Q4_0, INT8 and INT4 (per token and head) cache precisions on the GPU against the
oracle (needs an MI355X).

kv_type Q8_0 is the published llama.cpp block format that the operator's kv_type list names: per
token and KV head, 32-channel blocks with an fp16 scale max|x|/127 and int8 codes, ties away from
zero; Q4_0 its 4-bit sibling (scale m/-8 for the first largest-magnitude value m, codes
min(15, trunc(x/d + 8.5))); INT8 one fp32 scale max|x|/127 per token and KV head with Q8_0's
codes; INT4 one fp32 scale and one zero point per token and KV head (asymmetric, codes 0..15 packed
as Q4_0's).  The codes, scales and zero points must match the oracle bit for bit (both take the
rounding decisions in fp32); reps over the cached values are value-equal (Mean: relative 1e-4).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("no GPU", allow_module_level=True)

import block_sparse_kv_amd as kvs  # noqa: E402
from block_sparse_kv_amd import ops  # noqa: E402

import kvsynth  # noqa: E402
from oracle import kvs_oracle as orc  # noqa: E402
from parity import B, close_rel  # noqa: E402

DEV = "cuda"
REC = 128 * 128 + 128 * 4 * 2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def q8_cfg(Hkv=8, g=4, **kw):
    base = dict(num_q_heads=Hkv * g, num_kv_heads=Hkv, initial_len=128, local_len=256, topk=8,
                rep_method="quest", head_select_mode="separate", kv_type="q8_0")
    base.update(kw)
    return kvs.Config(**base)


def fp16_pool(n_phys, Hkv, seed):
    """Random fp16 tiles with the rows a quantizer can get wrong: an all-zero block, integer rows with
    +-127, exact ties at .5, very loud and very quiet blocks (fp16-subnormal scales)."""
    x = kvsynth.randn_fp16((n_phys, Hkv, B, 128), seed, DEV).float()
    g = torch.Generator(device="cpu")
    g.manual_seed(seed + 1)
    gain = torch.exp(torch.empty(n_phys, Hkv, B, 4).uniform_(-9.0, 7.0, generator=g)).to(DEV)
    x = (x.view(n_phys, Hkv, B, 4, 32) * gain[..., None]).view(n_phys, Hkv, B, 128)
    x[0, 0, 0, :32] = 0.0
    x[0, 0, 1, :] = torch.arange(-64, 64, dtype=torch.float32, device=DEV) * 2.0  # amax 128 in block 0
    x[0, 0, 2, :32] = torch.tensor([254.0, -127.0, 1.0, 3.0] + [0.0] * 28, device=DEV)  # ties
    x[0, 0, 3, :] = 127.0
    return x.to(torch.float16)


def split_q4(pool_q4):
    """[n][Hkv][9216] bytes -> codes uint8 [n][Hkv][128][128], scales fp16 [n][Hkv][128][4]."""
    a = pool_q4.cpu().numpy()
    w = a[..., : 128 * 64].copy().view(np.uint32).reshape(*a.shape[:2], 128, 16)
    codes = np.zeros((*a.shape[:2], 128, 128), dtype=np.uint8)
    for i in range(4):
        codes[..., 2 * i::8] = (w >> (4 * i)) & 0xF
        codes[..., 2 * i + 1::8] = (w >> (16 + 4 * i)) & 0xF
    scales = a[..., 128 * 64:].copy().view(np.float16).reshape(*a.shape[:2], 128, 4)
    return codes, scales


def split_records(pool_q8):
    """[n][Hkv][17408] bytes -> codes int8 [n][Hkv][128][128], scales fp16 [n][Hkv][128][4]."""
    a = pool_q8.cpu().numpy()
    codes = a[..., : 128 * 128].view(np.int8).reshape(*a.shape[:2], 128, 128)
    scales = a[..., 128 * 128:].copy().view(np.float16).reshape(*a.shape[:2], 128, 4)
    return codes, scales


@pytest.mark.parametrize("Hkv", [1, 8])
def test_quantize_bit_exact(Hkv):
    say(f"[case] q8 quantize Hkv={Hkv}")
    n_phys = 7
    c = q8_cfg(Hkv=Hkv, g=1)
    src = fp16_pool(n_phys, Hkv, kvsynth.mix_seed(401, Hkv))
    dst = ops.alloc_q8_pool(c, n_phys, DEV)
    dst.fill_(0xAB)
    ids = torch.tensor([5, 0, 3, 6], dtype=torch.int32)  # not every block, not in order
    ops.quantize_kv(c, src, ids, dst)
    torch.cuda.synchronize()
    got_c, got_s = split_records(dst)
    want_c, want_s = orc.quantize_q8_0(src.float().cpu().numpy())
    for p in range(n_phys):
        if p in ids.tolist():
            assert np.array_equal(got_c[p], want_c[p]), (p, np.argwhere(got_c[p] != want_c[p])[:4])
            assert np.array_equal(got_s[p].view(np.uint16), want_s[p].view(np.uint16)), p
        else:  # untouched
            assert np.all(dst[p].cpu().numpy() == 0xAB), p
    assert int(np.abs(want_c[ids.tolist()]).max()) == 127


@pytest.mark.parametrize("rep,rep_num", [("quest", 1), ("max", 1), ("mean", 1), ("fix", 8)])
def test_reps_over_q8_cache(rep, rep_num):
    say(f"[case] q8 reps {rep}/{rep_num}")
    n_phys, Hkv = 6, 8
    c = q8_cfg(Hkv=Hkv, rep_method=rep, rep_num=rep_num)
    src = fp16_pool(n_phys, Hkv, kvsynth.mix_seed(402, rep_num, len(rep)))
    kq = ops.alloc_q8_pool(c, n_phys, DEV)
    ids = torch.arange(n_phys, dtype=torch.int32)
    ops.quantize_kv(c, src, ids, kq)
    rp = ops.alloc_rep_pool(c, n_phys, DEV)
    ops.build_reps(c, kq, torch.tensor([4, 1, 2], dtype=torch.int32), rp)
    torch.cuda.synchronize()
    codes, scales = split_records(kq)
    for p in (4, 1, 2):
        K = orc.dequantize_q8_0(codes[p], scales[p]).transpose(1, 0, 2)  # [B tokens][Hkv][d]
        want = orc.stored_reps(orc.block_reps(K, B, rep, rep_num), rep)[0]  # [Hkv][R][d]
        got = rp[p].double().cpu().numpy()
        if rep == "mean":
            close_rel(got, want, np.abs(want).max(axis=-1, keepdims=True), f"q8 mean reps {p}")
        else:
            assert np.array_equal(got, want), (p, np.argwhere(got != want)[:4])


@pytest.mark.parametrize("Hkv", [1, 8])
def test_quantize_q4_bit_exact(Hkv):
    say(f"[case] q4 quantize Hkv={Hkv}")
    n_phys = 7
    c = q8_cfg(Hkv=Hkv, g=1, kv_type="q4_0")
    src = fp16_pool(n_phys, Hkv, kvsynth.mix_seed(411, Hkv))
    src[1, 0, 5, :32] = torch.tensor([8.0, -8.0] + [0.0] * 30, dtype=torch.float16, device=DEV)  # tie
    dst = ops.alloc_q8_pool(c, n_phys, DEV)
    assert dst.shape[-1] == 9216
    dst.fill_(0xAB)
    ids = torch.tensor([5, 0, 1, 6], dtype=torch.int32)
    ops.quantize_kv(c, src, ids, dst)
    torch.cuda.synchronize()
    got_c, got_s = split_q4(dst)
    want_c, want_s = orc.quantize_q4_0(src.float().cpu().numpy())
    for p in range(n_phys):
        if p in ids.tolist():
            assert np.array_equal(got_c[p], want_c[p]), (p, np.argwhere(got_c[p] != want_c[p])[:4])
            assert np.array_equal(got_s[p].view(np.uint16), want_s[p].view(np.uint16)), p
        else:
            assert np.all(dst[p].cpu().numpy() == 0xAB), p


def split_i8(pool_i8):
    """[n][Hkv][16896] bytes -> codes int8 [n][Hkv][128][128], scales fp32 [n][Hkv][128]."""
    a = pool_i8.cpu().numpy()
    codes = a[..., : 128 * 128].view(np.int8).reshape(*a.shape[:2], 128, 128)
    scales = a[..., 128 * 128:].copy().view(np.float32).reshape(*a.shape[:2], 128)
    return codes, scales


@pytest.mark.parametrize("Hkv", [1, 8])
def test_quantize_int8_pth_bit_exact(Hkv):
    say(f"[case] int8 per-token-head quantize Hkv={Hkv}")
    n_phys = 7
    c = q8_cfg(Hkv=Hkv, g=1, kv_type="int8_pth")
    src = fp16_pool(n_phys, Hkv, kvsynth.mix_seed(421, Hkv))
    src[2, 0, 9, :] = 0.0  # an all-zero row
    dst = ops.alloc_q8_pool(c, n_phys, DEV)
    assert dst.shape[-1] == 16896
    dst.fill_(0xAB)
    ids = torch.tensor([5, 0, 2, 6], dtype=torch.int32)
    ops.quantize_kv(c, src, ids, dst)
    torch.cuda.synchronize()
    got_c, got_s = split_i8(dst)
    want_c, want_s = orc.quantize_int8_pth(src.float().cpu().numpy())
    for p in range(n_phys):
        if p in ids.tolist():
            assert np.array_equal(got_c[p], want_c[p]), (p, np.argwhere(got_c[p] != want_c[p])[:4])
            assert np.array_equal(got_s[p].view(np.uint32), want_s[p].view(np.uint32)), p
        else:
            assert np.all(dst[p].cpu().numpy() == 0xAB), p
    assert float(got_s[2, 0, 9]) == 0.0 and not got_c[2, 0, 9].any()


@pytest.mark.parametrize("rep,rep_num", [("quest", 1), ("max", 1), ("mean", 1), ("fix", 8)])
def test_reps_over_int8_pth_cache(rep, rep_num):
    say(f"[case] int8 per-token-head reps {rep}/{rep_num}")
    n_phys, Hkv = 6, 8
    c = q8_cfg(Hkv=Hkv, rep_method=rep, rep_num=rep_num, kv_type="int8_pth")
    src = fp16_pool(n_phys, Hkv, kvsynth.mix_seed(422, rep_num, len(rep)))
    kq = ops.alloc_q8_pool(c, n_phys, DEV)
    ops.quantize_kv(c, src, torch.arange(n_phys, dtype=torch.int32), kq)
    rp = ops.alloc_rep_pool(c, n_phys, DEV)
    ops.build_reps(c, kq, torch.tensor([4, 1, 2], dtype=torch.int32), rp)
    torch.cuda.synchronize()
    codes, scales = split_i8(kq)
    for p in (4, 1, 2):
        K = orc.dequantize_int8_pth(codes[p], scales[p]).transpose(1, 0, 2)
        want = orc.stored_reps(orc.block_reps(K, B, rep, rep_num), rep)[0]
        got = rp[p].double().cpu().numpy()
        if rep == "mean":
            close_rel(got, want, np.abs(want).max(axis=-1, keepdims=True), f"int8 mean reps {p}")
        else:
            assert np.array_equal(got, want), (p, np.argwhere(got != want)[:4])


@pytest.mark.parametrize("rep,rep_num", [("quest", 1), ("mean", 1), ("fix", 4)])
def test_reps_over_q4_cache(rep, rep_num):
    say(f"[case] q4 reps {rep}/{rep_num}")
    n_phys, Hkv = 6, 8
    c = q8_cfg(Hkv=Hkv, rep_method=rep, rep_num=rep_num, kv_type="q4_0")
    src = fp16_pool(n_phys, Hkv, kvsynth.mix_seed(412, rep_num, len(rep)))
    kq = ops.alloc_q8_pool(c, n_phys, DEV)
    ops.quantize_kv(c, src, torch.arange(n_phys, dtype=torch.int32), kq)
    rp = ops.alloc_rep_pool(c, n_phys, DEV)
    ops.build_reps(c, kq, torch.tensor([4, 1, 2], dtype=torch.int32), rp)
    torch.cuda.synchronize()
    codes, scales = split_q4(kq)
    for p in (4, 1, 2):
        K = orc.dequantize_q4_0(codes[p], scales[p]).transpose(1, 0, 2)
        want = orc.stored_reps(orc.block_reps(K, B, rep, rep_num), rep)[0]
        got = rp[p].double().cpu().numpy()
        if rep == "mean":
            close_rel(got, want, np.abs(want).max(axis=-1, keepdims=True), f"q4 mean reps {p}")
        else:
            assert np.array_equal(got, want), (p, np.argwhere(got != want)[:4])


def split_i4(pool_i4):
    """[n][Hkv][8832] bytes -> codes uint8 [n][Hkv][128][128] (Q4_0's packing), scales fp32
    [n][Hkv][128], zero points uint8 [n][Hkv][128]."""
    a = pool_i4.cpu().numpy()
    w = a[..., : 128 * 64].copy().view(np.uint32).reshape(*a.shape[:2], 128, 16)
    codes = np.zeros((*a.shape[:2], 128, 128), dtype=np.uint8)
    for i in range(4):
        codes[..., 2 * i::8] = (w >> (4 * i)) & 0xF
        codes[..., 2 * i + 1::8] = (w >> (16 + 4 * i)) & 0xF
    scales = a[..., 128 * 64: 128 * 68].copy().view(np.float32).reshape(*a.shape[:2], 128)
    zeros = a[..., 128 * 68:].copy().reshape(*a.shape[:2], 128)
    return codes, scales, zeros


@pytest.mark.parametrize("Hkv", [1, 8])
def test_quantize_int4_pth_bit_exact(Hkv):
    say(f"[case] int4 per-token-head quantize Hkv={Hkv}")
    n_phys = 7
    c = q8_cfg(Hkv=Hkv, g=1, kv_type="int4_pth")
    src = fp16_pool(n_phys, Hkv, kvsynth.mix_seed(431, Hkv))
    src[2, 0, 9, :] = 0.0  # an all-zero row
    src[2, 0, 10, :] = torch.arange(128, dtype=torch.float32, device=DEV).to(torch.float16) / 8  # no negatives
    src[2, 0, 11, :] = -src[2, 0, 10, :]  # no positives
    row = torch.zeros(128, device=DEV)
    row[:8] = torch.tensor([20.0, -10.0, 1.0, 3.0, 5.0, -1.0, -3.0, 7.0], device=DEV)  # ties to even
    src[3, 0, 4, :] = row.to(torch.float16)
    row[:2] = torch.tensor([27.0, -3.0], device=DEV)  # a clamped code
    row[2:] = 0.0
    src[3, 0, 5, :] = row.to(torch.float16)
    dst = ops.alloc_q8_pool(c, n_phys, DEV)
    assert dst.shape[-1] == 8832
    dst.fill_(0xAB)
    ids = torch.tensor([5, 0, 2, 3, 6], dtype=torch.int32)
    ops.quantize_kv(c, src, ids, dst)
    torch.cuda.synchronize()
    got_c, got_s, got_z = split_i4(dst)
    want_c, want_s, want_z = orc.quantize_int4_pth(src.float().cpu().numpy())
    for p in range(n_phys):
        if p in ids.tolist():
            assert np.array_equal(got_c[p], want_c[p]), (p, np.argwhere(got_c[p] != want_c[p])[:4])
            assert np.array_equal(got_s[p].view(np.uint32), want_s[p].view(np.uint32)), p
            assert np.array_equal(got_z[p], want_z[p]), (p, np.argwhere(got_z[p] != want_z[p])[:4])
        else:
            assert np.all(dst[p].cpu().numpy() == 0xAB), p
    assert float(got_s[2, 0, 9]) == 0.0 and not got_c[2, 0, 9].any() and got_z[2, 0, 9] == 0
    assert got_z[2, 0, 10] == 0 and got_z[2, 0, 11] == 15
    assert got_z[3, 0, 4] == 5 and list(got_c[3, 0, 4, :8]) == [15, 0, 5, 7, 7, 5, 3, 9]
    assert got_z[3, 0, 5] == 2 and list(got_c[3, 0, 5, :2]) == [15, 0]


@pytest.mark.parametrize("rep,rep_num", [("quest", 1), ("max", 1), ("mean", 1), ("fix", 8)])
def test_reps_over_int4_pth_cache(rep, rep_num):
    say(f"[case] int4 per-token-head reps {rep}/{rep_num}")
    n_phys, Hkv = 6, 8
    c = q8_cfg(Hkv=Hkv, rep_method=rep, rep_num=rep_num, kv_type="int4_pth")
    src = fp16_pool(n_phys, Hkv, kvsynth.mix_seed(432, rep_num, len(rep)))
    kq = ops.alloc_q8_pool(c, n_phys, DEV)
    ops.quantize_kv(c, src, torch.arange(n_phys, dtype=torch.int32), kq)
    rp = ops.alloc_rep_pool(c, n_phys, DEV)
    ops.build_reps(c, kq, torch.tensor([4, 1, 2], dtype=torch.int32), rp)
    torch.cuda.synchronize()
    codes, scales, zeros = split_i4(kq)
    for p in (4, 1, 2):
        K = orc.dequantize_int4_pth(codes[p], scales[p], zeros[p]).transpose(1, 0, 2)
        want = orc.stored_reps(orc.block_reps(K, B, rep, rep_num), rep)[0]
        got = rp[p].double().cpu().numpy()
        if rep == "mean":
            close_rel(got, want, np.abs(want).max(axis=-1, keepdims=True), f"int4 mean reps {p}")
        else:
            assert np.array_equal(got, want), (p, np.argwhere(got != want)[:4])
