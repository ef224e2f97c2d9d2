"""Pins for the FP8 (OCP E4M3) cache oracle: oracle.fp8_decode, fp8_encode,
gqa_decode_fp8 and kv_append_fp8.

The 8-bit cache is the ranked next step after the bf16 path (an 8-bit cache
halves the bytes per token; "MHA -> MQA -> GQA -> MLA" and the
charlestar.github.io MLA page both name it, leaving the scale granularity
open).  Reading taken: E4M3 codes with one fp32 scale per tensor.

Independent checks:
  * torch's float8_e4m3fn conversions (a library routine) for every code and
    for in-range fp32 values, including exact ties;
  * closed forms of the format: 448 is the largest finite value, 2^-6 the
    smallest normal, 2^-9 the smallest subnormal, 1.0 = 0x38;
  * saturation beyond +-448 and NaN handling, written out;
  * the FP8 decode with power-of-two scales equals the (separately pinned)
    GQA oracle on the exactly dequantized fp32 cache; with any scale it
    equals torch's float64 attention on the dequantized values;
  * the FP8 append equals a numpy scatter of torch-converted codes.
"""
import numpy as np
import pytest
import torch

import oracle
from tests._util import bf16_bits, widen


def torch_codes(x):
    """torch's float32 -> E4M3 conversion, as codes (valid for |x| <= 448)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.fp8_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert nan.sum() == 2 and nan[0x7f] and nan[0xff]
    assert np.array_equal(mine[~nan], ref[~nan])


def test_decode_closed_forms():
    d = oracle.fp8_decode
    assert d(0x7e) == 448.0 and d(0xfe) == -448.0          # largest finite
    assert d(0x08) == 2.0 ** -6                             # smallest normal
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9   # subnormals
    assert d(0x38) == 1.0 and d(0xb8) == -1.0 and d(0x40) == 2.0
    assert d(0x00) == 0.0 and np.signbit(d(0x80))


def test_encode_round_trips_every_finite_code():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.fp8_decode(codes)
    fin = ~np.isnan(vals)
    assert np.array_equal(oracle.fp8_encode(vals[fin].astype(np.float32)), codes[fin])


def test_encode_matches_torch_in_range_including_ties():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(50000) * 40, rng.standard_normal(20000) * 1e-2,
                        rng.uniform(-448, 448, 20000)]).astype(np.float32)
    # exact midpoints between neighbouring finite codes (ties)
    v = oracle.fp8_decode(np.arange(0, 0x7e, dtype=np.uint8))
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    assert np.array_equal(oracle.fp8_encode(x), torch_codes(x))


def test_encode_ties_to_even_and_saturation():
    e = oracle.fp8_encode
    assert e(np.float32(1.0625)) == 0x38      # between 1.0 (m=0) and 1.125 (m=1): even m=0
    assert e(np.float32(1.1875)) == 0x3a      # between 1.125 (m=1) and 1.25 (m=2): even m=2
    assert e(np.float32(440.0)) == 0x7e       # 440 is 13.75 quanta of 32 -> 448
    for big in (448.0, 449.0, 464.0, 1e6, np.inf):
        assert e(np.float32(big)) == 0x7e and e(np.float32(-big)) == 0xfe
    assert e(np.float32(np.nan)) == 0x7f
    assert e(np.float32(2.0 ** -10)) == 0x00      # half the smallest subnormal: ties to even 0
    assert e(np.float32(3 * 2.0 ** -10)) == 0x02  # 1.5 quanta -> 2
    assert e(np.float32(-0.0)) == 0x80


def _fp8_case(B, h, h_kv, d, s, seed, k_scale, v_scale):
    rng = np.random.default_rng(seed)
    s_max = max(s)
    q = bf16_bits(rng.standard_normal((B, h, d)))
    K8 = oracle.fp8_encode(rng.standard_normal((B, s_max, h_kv, d)).astype(np.float32) / k_scale)
    V8 = oracle.fp8_encode(rng.standard_normal((B, s_max, h_kv, d)).astype(np.float32) / v_scale)
    return q, K8, V8, np.asarray(s, dtype=np.int32)


def test_fp8_decode_equals_gqa_oracle_on_dequantized_cache():
    k_scale, v_scale = 0.25, 2.0 ** -3     # powers of two: dequantized values exact in fp32
    q, K8, V8, s = _fp8_case(2, 8, 2, 64, [37, 70], 3, k_scale, v_scale)
    out, lse = oracle.gqa_decode_fp8(q, K8, V8, k_scale, v_scale, s)
    Kf = (oracle.fp8_decode(K8) * k_scale).astype(np.float32)
    Vf = (oracle.fp8_decode(V8) * v_scale).astype(np.float32)
    qf = widen(q).astype(np.float32)
    ref, rlse = oracle.gqa_decode(qf, Kf, Vf, s, 4)
    assert np.abs(out - ref).max() <= 1e-12 and np.abs(lse - rlse).max() <= 1e-12


def test_fp8_decode_matches_torch_attention():
    k_scale, v_scale = 0.0371, 0.0593
    q, K8, V8, s = _fp8_case(3, 16, 4, 128, [1, 33, 90], 4, k_scale, v_scale)
    out, lse = oracle.gqa_decode_fp8(q, K8, V8, k_scale, v_scale, s)
    qd = widen(q)
    Kd = oracle.fp8_decode(K8) * float(np.float32(k_scale))
    Vd = oracle.fp8_decode(V8) * float(np.float32(v_scale))
    g = 4
    for bi in range(3):
        n = int(s[bi])
        qt = torch.from_numpy(qd[bi]).unsqueeze(1)
        kt = torch.from_numpy(Kd[bi, :n]).permute(1, 0, 2).repeat_interleave(g, 0)
        vt = torch.from_numpy(Vd[bi, :n]).permute(1, 0, 2).repeat_interleave(g, 0)
        z = (qt @ kt.transpose(1, 2)) / np.sqrt(128)
        ref = (torch.softmax(z, -1) @ vt).squeeze(1).numpy()
        rl = torch.logsumexp(z, -1).squeeze(1).numpy()
        assert np.abs(out[bi] - ref).max() <= 1e-11
        assert np.abs(lse[bi] - rl).max() <= 1e-11


def test_fp8_append_matches_numpy_scatter():
    rng = np.random.default_rng(5)
    B, s_max, h_kv, d = 4, 12, 2, 64
    k_scale, v_scale = 0.02, 0.5
    ck = rng.integers(0, 255, (B, s_max, h_kv, d), dtype=np.uint8)
    cv = rng.integers(0, 255, (B, s_max, h_kv, d), dtype=np.uint8)
    kn = bf16_bits(rng.standard_normal((B, h_kv, d)) * 3)
    vn = bf16_bits(rng.standard_normal((B, h_kv, d)) * 300)   # some saturate (|x|/0.5 > 448)
    pos = np.array([0, 5, 11, 7], dtype=np.int32)
    nk, nv = oracle.kv_append_fp8(ck, cv, kn, vn, k_scale, v_scale, pos)
    ek, ev = ck.copy(), cv.copy()
    ik, iv = np.float32(1) / np.float32(k_scale), np.float32(1) / np.float32(v_scale)
    for bi in range(B):
        yk = widen(kn[bi]).astype(np.float32) * ik
        yv = widen(vn[bi]).astype(np.float32) * iv
        ek[bi, pos[bi]] = torch_codes(np.clip(yk, -448, 448))
        ev[bi, pos[bi]] = torch_codes(np.clip(yv, -448, 448))
    assert np.array_equal(nk, ek) and np.array_equal(nv, ev)


def paged_fp8_case(seed, B=3, h=8, h_kv=2, d=64, s=(40, 17, 70)):
    rng = np.random.default_rng(seed)
    nblk = [(n + 15) // 16 for n in s]
    N = sum(nblk)
    perm = rng.permutation(N)
    bt = np.full((B, max(nblk)), -1, np.int32)
    k = 0
    for bi in range(B):
        for jb in range(nblk[bi]):
            bt[bi, jb] = perm[k]
            k += 1
    q = bf16_bits(rng.standard_normal((B, h, d)))
    # per (page, KV head) powers of two, so that dequantised values are exact in fp32
    ks = (2.0 ** rng.integers(-8, -2, size=(N, h_kv))).astype(np.float32)
    vs = (2.0 ** rng.integers(-8, -2, size=(N, h_kv))).astype(np.float32)
    K8 = oracle.fp8_encode((rng.standard_normal((N, 16, h_kv, d)) / ks[:, None, :, None]).astype(np.float32))
    V8 = oracle.fp8_encode((rng.standard_normal((N, 16, h_kv, d)) / vs[:, None, :, None]).astype(np.float32))
    return q, K8, V8, ks, vs, np.array(s, np.int32), bt


def test_per_page_scales_equal_the_dequantised_paged_oracle():
    q, K8, V8, ks, vs, s, bt = paged_fp8_case(7)
    out, lse = oracle.gqa_decode_fp8_paged_scales(q, K8, V8, ks, vs, s, bt)
    Kd = (oracle.fp8_decode(K8) * ks[:, None, :, None]).astype(np.float32)
    Vd = (oracle.fp8_decode(V8) * vs[:, None, :, None]).astype(np.float32)
    ro, rl = oracle.gqa_decode(widen(q).astype(np.float32), Kd, Vd, s, 4, block_table=bt)
    assert np.max(np.abs(out - ro)) < 1e-12 and np.max(np.abs(lse - rl)) < 1e-12


def test_uniform_per_page_scales_equal_the_per_tensor_oracle():
    q, K8, V8, ks, vs, s, bt = paged_fp8_case(8)
    ks[:] = 0.03
    vs[:] = 0.07
    out, lse = oracle.gqa_decode_fp8_paged_scales(q, K8, V8, ks, vs, s, bt)
    ro, rl = oracle.gqa_decode_fp8(q, K8, V8, 0.03, 0.07, s, block_table=bt)
    assert np.array_equal(out, ro) and np.array_equal(lse, rl)


def test_per_page_append_uses_its_pages_scale():
    rng = np.random.default_rng(9)
    q, K8, V8, ks, vs, s, bt = paged_fp8_case(9)
    B, h_kv, d = 3, 2, 64
    kn = bf16_bits(rng.standard_normal((B, h_kv, d)) * 0.3)
    vn = bf16_bits(rng.standard_normal((B, h_kv, d)) * 0.3)
    pos = np.array([39, 0, 69], np.int32)
    ck, cv = oracle.kv_append_fp8_paged_scales(K8, V8, kn, vn, ks, vs, pos, bt)
    wk, wv = K8.copy(), V8.copy()
    for bi in range(B):
        blk = bt[bi, pos[bi] // 16]
        for j in range(h_kv):
            ik = np.float32(1.0) / ks[blk, j]
            iv = np.float32(1.0) / vs[blk, j]
            xk = torch.from_numpy(widen(kn[bi, j]).astype(np.float32) * ik)
            xv = torch.from_numpy(widen(vn[bi, j]).astype(np.float32) * iv)
            wk[blk, pos[bi] % 16, j] = xk.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            wv[blk, pos[bi] % 16, j] = xv.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ck, wk) and np.array_equal(cv, wv)
