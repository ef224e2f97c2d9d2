"""GPU parity of the FP8 (OCP E4M3) cache path against the CPU oracle.

attn_decode_gqa_fp8 is compared element by element with
oracle.gqa_decode_fp8 on the same codes and scales (small cases spanning
several tiles and ragged tails, every group size of the matrix-core kernel,
paged with a shuffled table, split contexts), and on sampled KV-head groups
at the Llama-3-8B shape.  The codes widen to bf16 exactly, so the tolerances
are those of the bf16 path (max-abs <= 2e-2, mean-abs <= 2e-3, rel-RMS <=
1e-2).  kv_cache_append_fp8 is bit-exact against oracle.kv_append_fp8,
including ties, saturation, NaN and signed zero.
"""
import numpy as np
import pytest
import torch

import decode_attention_kv_attn_amd as A
import oracle
import synth
from tests._gpu import assert_close, assert_lse_close, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"
KS, VS = 1.0 / 64, 0.0123   # per-tensor scales (one power of two, one not)


def run_fp8(B, h, h_kv, d_h, s, seed, paged=False, k_scale=KS, v_scale=VS):
    sh = synth.GqaShape("t", B=B, h=h, h_kv=h_kv, d_h=d_h, b=2, s=tuple(s), paged=paged, seed=seed)
    print(f"[fp8] B={B} h={h} h_kv={h_kv} d_h={d_h} s={list(s)[:6]} paged={paged}", flush=True)
    d = synth.draw_gqa_fp8(sh, k_scale, v_scale, device=DEV)
    bt = d.get("block_table")
    out, lse = A.decode_gqa_fp8(d["q"], d["K8"], d["V8"], k_scale, v_scale, d["s"], block_table=bt,
                                s_max=sh.s_max)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.gqa_decode_fp8(synth.host_bits(d["q"]), synth.host_bits(d["K8"]),
                                         synth.host_bits(d["V8"]), k_scale, v_scale, d["s_host"],
                                         block_table=d.get("block_table_host"))
    assert_close(to_f64(out), ref, 2, "out")
    assert_lse_close(to_f64(lse), ref_lse, 2, "lse")


@pytest.mark.parametrize("h,h_kv", [(8, 8), (16, 4), (32, 8), (16, 2), (64, 1), (12, 4), (40, 2)])
@pytest.mark.parametrize("d_h", [64, 128])
def test_fp8_group_sizes(h, h_kv, d_h):
    run_fp8(3, h, h_kv, d_h, (1, 77, 300), seed=h * 10 + h_kv)


@pytest.mark.parametrize("s", [(0, 5), (0, 0), (1, 1), (31, 33), (32, 64), (63, 65)])
def test_fp8_ragged_and_degenerate(s):
    run_fp8(2, 16, 2, 128, s, seed=5)


def test_fp8_paged_shuffled():
    run_fp8(4, 32, 8, 128, (16, 17, 250, 1000), seed=6, paged=True)


def test_fp8_split_context():
    # one sequence of 9000 tokens over one KV head: several splits and the merge
    run_fp8(1, 8, 1, 128, (9000,), seed=7)


def test_fp8_scales_enter_scores_and_values():
    run_fp8(2, 16, 4, 128, (200, 65), seed=8, k_scale=0.037, v_scale=2.5)


def test_fp8_llama3_8b_shape_sampled():
    sh = synth.GqaShape("t", B=64, h=32, h_kv=8, d_h=128, b=2, s=(4096,) * 64, seed=2)
    d = synth.draw_gqa_fp8(sh, KS, VS, device=DEV)
    out, lse = A.decode_gqa_fp8(d["q"], d["K8"], d["V8"], KS, VS, d["s"])
    torch.cuda.synchronize()
    g = 4
    for (bi, j) in [(0, 0), (17, 3), (63, 7)]:
        q = synth.host_bits(d["q"][bi:bi + 1, j * g:(j + 1) * g])
        K = synth.host_bits(d["K8"][bi, :, j])[None, :, None, :]
        V = synth.host_bits(d["V8"][bi, :, j])[None, :, None, :]
        ref, rl = oracle.gqa_decode_fp8(q, K, V, KS, VS, np.array([4096], np.int32))
        assert_close(to_f64(out[bi, j * g:(j + 1) * g]), ref[0], 2, f"b={bi} j={j}")
        assert_lse_close(to_f64(lse[bi, j * g:(j + 1) * g]), rl[0], 2, f"b={bi} j={j}")


def test_fp8_rejects_bad_arguments():
    q = torch.zeros(1, 128, 128, dtype=torch.bfloat16, device=DEV)
    K8 = torch.zeros(1, 16, 1, 128, dtype=torch.uint8, device=DEV)
    s = torch.tensor([16], dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    rc = A.attn_decode_gqa_fp8(out, None, q, K8, K8, KS, VS, s, None, 0, 16, 0, 1, 16, 128, 1,
                               128, 0.0, None, 0, check=False)
    assert rc == A.ATTN_ENOTSUP   # g = 128 > 64
    rc = A.attn_decode_gqa_fp8(out, None, q[:, :8], K8, K8, 0.0, VS, s, None, 0, 16, 0, 1, 16, 8,
                               1, 128, 0.0, None, 0, check=False)
    assert rc == A.ATTN_EINVAL    # non-positive scale


def special_rows(B, h_kv, d_h, scale):
    """bf16 rows with ties, saturating values, NaN, infinities, signed zeros."""
    x = torch.randn(B, h_kv, d_h, device=DEV) * 40 * scale
    flat = x.view(-1)
    codes = torch.arange(0, 0x7e, device=DEV, dtype=torch.uint8).view(torch.float8_e4m3fn).float()
    mids = (codes[:-1] + codes[1:]) / 2 * scale          # ties (exact in bf16 where representable)
    n = min(mids.numel(), flat.numel() // 4)
    flat[:n] = mids[:n]
    flat[n:n + 8] = torch.tensor([500.0, -1e4, float("inf"), float("-inf"), float("nan"), 0.0, -0.0,
                                  448.0], device=DEV) * scale
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("paged", [False, True])
def test_fp8_append_bit_exact(paged):
    B, s_max, h_kv, d_h = 5, 40, 8, 128
    k_scale, v_scale = 0.02, 0.5
    sh = synth.GqaShape("t", B=B, h=h_kv, h_kv=h_kv, d_h=d_h, b=2, s=(s_max,) * B, paged=paged,
                        seed=23)
    d = synth.draw_gqa_fp8(sh, k_scale, v_scale, device=DEV)
    kn, vn = special_rows(B, h_kv, d_h, k_scale), special_rows(B, h_kv, d_h, v_scale)
    pos = torch.tensor([0, 39, 7, 16, 31], dtype=torch.int32, device=DEV)
    bt = d.get("block_table")
    refK, refV = oracle.kv_append_fp8(synth.host_bits(d["K8"]), synth.host_bits(d["V8"]),
                                      synth.host_bits(kn), synth.host_bits(vn), k_scale, v_scale,
                                      pos.cpu().numpy(), block_table=d.get("block_table_host"))
    A.kv_cache_append_fp8(d["K8"], d["V8"], kn, vn, k_scale, v_scale, pos, bt,
                          0 if bt is None else bt.shape[1], 16,
                          0 if bt is None else d["K8"].shape[0], B, s_max, h_kv, d_h)
    torch.cuda.synchronize()
    assert np.array_equal(synth.host_bits(d["K8"]), refK)
    assert np.array_equal(synth.host_bits(d["V8"]), refV)


def test_fp8_paged_mixed_lengths_many_splits():
    run_fp8(8, 32, 8, 128, (0, 5000, 1, 700, 0, 9000, 33, 4097), seed=18, paged=True)


def page_scaled_pool(sh, seed):
    """Paged E4M3 pools with one power-of-two-free scale per (page, KV head)."""
    d = synth.draw_gqa(sh, device=DEV)   # bf16 pools and table
    g = torch.Generator(device=DEV).manual_seed(seed)
    N = d["K"].shape[0]
    ks = (torch.rand((N, sh.h_kv), generator=g, device=DEV) * 0.05 + 0.005).float()
    vs = (torch.rand((N, sh.h_kv), generator=g, device=DEV) * 0.05 + 0.005).float()
    K8 = (d["K"].float() / ks[:, None, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    V8 = (d["V"].float() / vs[:, None, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    return d, K8.contiguous(), V8.contiguous(), ks, vs


@pytest.mark.parametrize("B,h,h_kv,d_h,s", [(4, 32, 8, 128, (1, 16, 17, 500)),
                                            (3, 16, 2, 64, (5, 300, 1000)),
                                            (8, 64, 8, 128, (0, 5000, 1, 700, 0, 9000, 33, 4097))])
def test_fp8_per_page_scales(B, h, h_kv, d_h, s):
    sh = synth.GqaShape("t", B=B, h=h, h_kv=h_kv, d_h=d_h, b=2, s=s, paged=True, seed=B * 10 + h)
    print(f"[fp8-page-scales] B={B} h={h} h_kv={h_kv} d_h={d_h}", flush=True)
    d, K8, V8, ks, vs = page_scaled_pool(sh, seed=B + h)
    bt = d["block_table"]
    out = torch.empty_like(d["q"])
    lse = torch.empty((B, h), dtype=torch.float32, device=DEV)
    wsb = A.attn_decode_workspace_bytes(0, B, sh.s_max, h, h_kv, d_h)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=DEV)
    A.attn_decode_gqa_fp8_paged_scales(out, lse, d["q"], K8, V8, ks, vs, d["s"], bt, bt.shape[1], 16,
                                       K8.shape[0], B, sh.s_max, h, h_kv, d_h, 0.0, ws, wsb)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.gqa_decode_fp8_paged_scales(synth.host_bits(d["q"]), synth.host_bits(K8),
                                                      synth.host_bits(V8), ks.cpu().numpy(),
                                                      vs.cpu().numpy(), d["s_host"],
                                                      d["block_table_host"])
    assert_close(to_f64(out), ref, 2, "out")
    assert_lse_close(to_f64(lse), ref_lse, 2, "lse")


def test_fp8_per_page_scales_uniform_equal_per_tensor_call():
    # the same scale on every page: the same kernel arithmetic as the per-tensor entry point
    sh = synth.GqaShape("t", B=3, h=32, h_kv=8, d_h=128, b=2, s=(40, 700, 3000), paged=True, seed=77)
    d, _, _, ks, vs = page_scaled_pool(sh, seed=77)
    ks.fill_(0.02)
    vs.fill_(0.03)
    K8 = synth.fp8_codes(d["K"], 0.02).contiguous()
    V8 = synth.fp8_codes(d["V"], 0.03).contiguous()
    bt = d["block_table"]
    o1, l1 = A.decode_gqa_fp8(d["q"], K8, V8, 0.02, 0.03, d["s"], block_table=bt, s_max=sh.s_max)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    wsb = A.attn_decode_workspace_bytes(0, 3, sh.s_max, 32, 8, 128)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=DEV)
    A.attn_decode_gqa_fp8_paged_scales(o2, l2, d["q"], K8, V8, ks, vs, d["s"], bt, bt.shape[1], 16,
                                       K8.shape[0], 3, sh.s_max, 32, 8, 128, 0.0, ws, wsb)
    torch.cuda.synchronize()
    assert_close(to_f64(o2), to_f64(o1), 2, "out")
    # the per-tensor path sums the bf16-rounded weights, the per-page path the
    # unrounded ones (its P carries the page's V scale): lse within bf16 rounding
    assert_lse_close(to_f64(l2), to_f64(l1), 2, "lse")


def test_fp8_per_page_append_bit_exact():
    rng = np.random.default_rng(78)
    B, h_kv, d_h, nblk = 5, 4, 128, 12
    bt = rng.permutation(nblk).astype(np.int32)[:10].reshape(5, 2)
    pool_k = torch.from_numpy(rng.integers(0, 256, size=(nblk, 16, h_kv, d_h), dtype=np.uint8)).to(DEV)
    pool_v = torch.from_numpy(rng.integers(0, 256, size=(nblk, 16, h_kv, d_h), dtype=np.uint8)).to(DEV)
    ks = torch.from_numpy((rng.random((nblk, h_kv)) * 0.1 + 0.01).astype(np.float32)).to(DEV)
    vs = torch.from_numpy((rng.random((nblk, h_kv)) * 0.1 + 0.01).astype(np.float32)).to(DEV)
    kn = torch.from_numpy(rng.standard_normal((B, h_kv, d_h)).astype(np.float32) * 2).to(torch.bfloat16)
    vn = torch.from_numpy(rng.standard_normal((B, h_kv, d_h)).astype(np.float32) * 2).to(torch.bfloat16)
    kn[0, 0, 0] = float("nan")
    kn[1, 1, 1] = 1e5
    pos = np.array([0, 31, 16, 15, 7], np.int32)
    hk, hv = synth.host_bits(pool_k), synth.host_bits(pool_v)
    A.kv_cache_append_fp8_paged_scales(pool_k, pool_v, kn.to(DEV), vn.to(DEV), ks, vs,
                                       torch.from_numpy(pos).to(DEV), torch.from_numpy(bt).to(DEV), 2,
                                       16, nblk, B, 32, h_kv, d_h)
    torch.cuda.synchronize()
    wk, wv = oracle.kv_append_fp8_paged_scales(hk, hv, synth.host_bits(kn), synth.host_bits(vn),
                                               ks.cpu().numpy(), vs.cpu().numpy(), pos, bt)
    assert np.array_equal(synth.host_bits(pool_k), wk) and np.array_equal(synth.host_bits(pool_v), wv)


def test_fp8_per_page_scales_rejects_bad_arguments():
    out = torch.empty((1, 8, 64), dtype=torch.bfloat16, device=DEV)
    fake = out.data_ptr()
    kw = dict(out=out, lse=None, q=out, cache_k=fake, cache_v=fake, k_scales=fake, v_scales=fake,
              s=fake, block_table=fake, max_blocks=1, block_size=16, num_blocks=1, B=1, s_max=16,
              h=8, h_kv=2, d_h=64, scale=0.0, workspace=None, workspace_bytes=0, check=False)
    assert A.attn_decode_gqa_fp8_paged_scales(**{**kw, "k_scales": None}) == A.ATTN_EINVAL
    assert A.attn_decode_gqa_fp8_paged_scales(**{**kw, "block_table": None}) == A.ATTN_EINVAL
