"""Pins for the oracle's MLA decode over an FP8 latent cache
(oracle.mla_absorbed_fp8) and its append (oracle.kv_append_mla_fp8).

  * With power-of-two scales every dequantised element is exact in fp32, so
    the FP8 decode must equal the (pinned) absorbed oracle run on the
    dequantised fp32 cache, and the explicit K/V expansion of it.
  * With unrelated scales for the latent and rotary parts (0.013 and 2.7),
    applying either scale to the wrong part, or one scale to both, moves the
    result far outside the fp32-dequantisation tolerance used here.
  * The append encodes each part with its own reciprocal scale exactly as
    torch's float8_e4m3fn conversion does, scattered by numpy.
  * Per-page scales (one latent and one rotary scale per page of the paged
    pool; llms.blog MLA page, "High-Throughput Serving Kernels: FlashMLA and
    SGLang", per-block scaling factors): equal scales on every page give the
    per-tensor decode bit for bit; distinct power-of-two scales per page, over
    a shuffled table, give the bf16 oracle on the dequantised pool bit for
    bit (so a page looked up by its logical rather than physical index
    fails); the per-page append equals the per-tensor append wherever a
    sequence's pages share one scale pair, and torch's conversion per page.
"""
import numpy as np
import torch

import oracle
from tests._util import bf16_bits, widen

D_C, D_R, D_NOPE, D_V = 512, 64, 128, 128


def draw(B, h, s, cs, rs, seed, s_max=None):
    rng = np.random.default_rng(seed)
    s_max = s_max or max(s)
    qn = bf16_bits(rng.standard_normal((B, h, D_NOPE)))
    qr = bf16_bits(rng.standard_normal((B, h, D_R)))
    wuk = bf16_bits(rng.standard_normal((h, D_NOPE, D_C)) / np.sqrt(D_C))
    wuv = bf16_bits(rng.standard_normal((h, D_V, D_C)) / np.sqrt(D_C))
    lat = rng.standard_normal((B, s_max, D_C + D_R))
    lat[..., :D_C] /= cs
    lat[..., D_C:] /= rs
    codes = oracle.fp8_encode(lat.astype(np.float32))
    return qn, qr, wuk, wuv, codes, np.array(s, np.int32)


def dequant(codes, cs, rs):
    x = oracle.fp8_decode(codes).astype(np.float64)
    x[..., :D_C] *= cs
    x[..., D_C:] *= rs
    return x


def test_power_of_two_scales_equal_the_dequantised_oracle():
    cs, rs = 2.0 ** -6, 0.5
    qn, qr, wuk, wuv, codes, s = draw(2, 8, (40, 7), cs, rs, seed=1)
    out, ul, lse = oracle.mla_absorbed_fp8(qn, qr, wuk, wuv, codes, cs, rs, s)
    f32 = lambda a: widen(a).astype(np.float32)
    deq = dequant(codes, cs, rs).astype(np.float32)
    ro, ru, rl = oracle.mla_absorbed(f32(qn), f32(qr), f32(wuk), f32(wuv), deq, s, b=4)
    assert np.max(np.abs(out - ro)) < 1e-12
    assert np.max(np.abs(ul - ru)) < 1e-12
    assert np.max(np.abs(lse - rl)) < 1e-12
    eo, el = oracle.mla_explicit(f32(qn), f32(qr), f32(wuk), f32(wuv), deq, s, b=4)
    assert np.max(np.abs(out - eo)) <= 1e-10 * max(1.0, np.max(np.abs(eo)))
    assert np.max(np.abs(lse - el)) < 1e-10


def test_each_part_takes_its_own_scale():
    cs, rs = 0.013, 2.7
    qn, qr, wuk, wuv, codes, s = draw(2, 4, (30, 5), cs, rs, seed=2)
    out, ul, lse = oracle.mla_absorbed_fp8(qn, qr, wuk, wuv, codes, cs, rs, s)
    f32 = lambda a: widen(a).astype(np.float32)

    def ref(c_s, r_s):
        deq = dequant(codes, c_s, r_s).astype(np.float32)
        return oracle.mla_absorbed(f32(qn), f32(qr), f32(wuk), f32(wuv), deq, s, b=4)

    ro, ru, rl = ref(cs, rs)
    # fp32 rounding of the dequantised cache bounds the agreement
    assert np.max(np.abs(out - ro)) < 1e-5 and np.max(np.abs(lse - rl)) < 1e-4
    for wrong in ((rs, cs), (cs, cs), (rs, rs)):
        wo, _, wl = ref(*wrong)
        assert np.max(np.abs(lse - wl)) > 1e-2


def test_paged_equals_contiguous():
    cs, rs = 0.02, 0.05
    qn, qr, wuk, wuv, codes, s = draw(2, 4, (20, 35), cs, rs, seed=3, s_max=48)
    # scatter the rows into a shuffled pool of 16-row blocks
    rng = np.random.default_rng(3)
    nblk = [(n + 15) // 16 for n in s]
    perm = rng.permutation(sum(nblk))
    pool = np.zeros((sum(nblk), 16, D_C + D_R), np.uint8)
    bt = np.full((2, 3), -1, np.int32)
    k = 0
    for bi in range(2):
        for j in range(nblk[bi]):
            bt[bi, j] = perm[k]
            rows = codes[bi, 16 * j:16 * j + 16]
            pool[perm[k], :rows.shape[0]] = rows
            k += 1
    a = oracle.mla_absorbed_fp8(qn, qr, wuk, wuv, codes, cs, rs, s)
    b = oracle.mla_absorbed_fp8(qn, qr, wuk, wuv, pool, cs, rs, s, block_table=bt)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_append_encodes_each_part_with_its_scale():
    cs, rs = 0.03, 0.7
    rng = np.random.default_rng(4)
    B, s_max = 3, 10
    cache = rng.integers(0, 256, size=(B, s_max, D_C + D_R), dtype=np.uint8)
    kv = bf16_bits(rng.standard_normal((B, D_C + D_R)) * 5)
    pos = np.array([0, 9, 4], np.int32)
    got = oracle.kv_append_mla_fp8(cache, kv, cs, rs, pos, D_C)
    want = cache.copy()
    x = torch.from_numpy(widen(kv).astype(np.float32))
    ic, ir = np.float32(1.0) / np.float32(cs), np.float32(1.0) / np.float32(rs)
    enc_c = (x[:, :D_C] * float(ic)).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    enc_r = (x[:, D_C:] * float(ir)).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for bi in range(B):
        want[bi, pos[bi], :D_C] = enc_c[bi]
        want[bi, pos[bi], D_C:] = enc_r[bi]
    assert np.array_equal(got, want)


def paged_pool(codes, s, seed):
    """Scatter contiguous rows [B, s_max, W] into a shuffled pool of 16-row
    pages; returns (pool, table)."""
    rng = np.random.default_rng(seed)
    B = codes.shape[0]
    nblk = [(n + 15) // 16 for n in s]
    perm = rng.permutation(sum(nblk))
    pool = np.zeros((sum(nblk), 16) + codes.shape[2:], codes.dtype)
    bt = np.full((B, max(nblk)), -1, np.int32)
    k = 0
    for bi in range(B):
        for j in range(nblk[bi]):
            bt[bi, j] = perm[k]
            rows = codes[bi, 16 * j:16 * j + 16]
            pool[perm[k], :rows.shape[0]] = rows
            k += 1
    return pool, bt


def test_page_scales_all_equal_give_the_per_tensor_decode():
    cs, rs = 0.013, 2.7
    qn, qr, wuk, wuv, codes, s = draw(3, 4, (20, 35, 1), cs, rs, seed=5, s_max=48)
    pool, bt = paged_pool(codes, s, 5)
    n = pool.shape[0]
    a = oracle.mla_absorbed_fp8(qn, qr, wuk, wuv, pool, cs, rs, s, block_table=bt)
    b = oracle.mla_absorbed_fp8_paged_scales(qn, qr, wuk, wuv, pool, np.full(n, cs, np.float32),
                                             np.full(n, rs, np.float32), s, bt)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_power_of_two_page_scales_equal_the_bf16_oracle_on_the_dequantised_pool():
    qn, qr, wuk, wuv, codes, s = draw(2, 8, (40, 23), 1.0, 1.0, seed=6, s_max=48)
    pool, bt = paged_pool(codes, s, 6)
    n = pool.shape[0]
    rng = np.random.default_rng(6)
    cs = (2.0 ** rng.integers(-8, -2, size=n)).astype(np.float32)   # distinct per page
    rs = (2.0 ** rng.integers(-3, 2, size=n)).astype(np.float32)
    out, ul, lse = oracle.mla_absorbed_fp8_paged_scales(qn, qr, wuk, wuv, pool, cs, rs, s, bt)
    deq = oracle.fp8_decode(pool).astype(np.float64)
    deq[..., :D_C] *= cs[:, None, None]
    deq[..., D_C:] *= rs[:, None, None]
    bits = bf16_bits(deq.astype(np.float32))
    assert np.array_equal(widen(bits), deq)          # exact in bf16
    ro, ru, rl = oracle.mla_absorbed(qn, qr, wuk, wuv, bits, s, block_table=bt)
    assert np.array_equal(out, ro) and np.array_equal(ul, ru) and np.array_equal(lse, rl)


def test_page_scale_append():
    rng = np.random.default_rng(7)
    B, nblk = 3, 6
    pool = rng.integers(0, 256, size=(nblk, 16, D_C + D_R), dtype=np.uint8)
    bt = np.array([[4, 1], [0, 5], [2, 3]], np.int32)
    kv = bf16_bits(rng.standard_normal((B, D_C + D_R)) * 5)
    pos = np.array([17, 3, 30], np.int32)   # pages 1, 0, 3
    cs = np.array([0.5, 0.03, 0.25, 0.011, 0.1, 0.07], np.float32)
    rs = np.array([0.2, 0.7, 1.5, 0.031, 0.9, 0.4], np.float32)
    got = oracle.kv_append_mla_fp8_paged_scales(pool, kv, cs, rs, pos, D_C, bt)
    want = pool.copy()
    x = torch.from_numpy(widen(kv).astype(np.float32))
    for bi in range(B):
        blk = bt[bi, pos[bi] // 16]
        ic, ir = np.float32(1.0) / cs[blk], np.float32(1.0) / rs[blk]
        want[blk, pos[bi] % 16, :D_C] = (x[bi, :D_C] * float(ic)).clamp(-448, 448).to(
            torch.float8_e4m3fn).view(torch.uint8).numpy()
        want[blk, pos[bi] % 16, D_C:] = (x[bi, D_C:] * float(ir)).clamp(-448, 448).to(
            torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)
    # sequence 1's pages share one pair with each other: the per-tensor append agrees
    same = np.array([0.03, 0.03, 0.03, 0.03, 0.03, 0.03], np.float32)
    a = oracle.kv_append_mla_fp8_paged_scales(pool, kv, same, same * 10, pos, D_C, bt)
    b = oracle.kv_append_mla_fp8(pool, kv, 0.03, np.float32(0.03) * np.float32(10), pos, D_C,
                                 block_table=bt)
    assert np.array_equal(a, b)
