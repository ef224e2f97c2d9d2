"""GPU parity of attn_decode_gqa_multi(_fp8) -- q_len new tokens per
sequence, causal among them -- against the oracle's multi-token decode.

Small cases compare every element (several tiles, ragged tails, sequences
shorter than q_len, splits, 64-row blocks, paged tables); the full-size
Llama-3 layers with 4 drafted tokens compare sampled KV-head groups in the
benchmark's launch configuration.  Tolerances: the bf16 bar (max-abs <= 2e-2,
mean-abs <= 2e-3, rel-RMS <= 1e-2), lse as the single-token tests.
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


def draw(B, T, h, h_kv, d_h, s, seed, paged=False, fp8=None):
    sh = synth.GqaShape("t", B=B, h=h, h_kv=h_kv, d_h=d_h, b=2, s=tuple(s), paged=paged, seed=seed)
    if fp8 is None:
        d = synth.draw_gqa(sh, device=DEV)
    else:
        d = synth.draw_gqa_fp8(sh, fp8[0], fp8[1], device=DEV)
        d["K"], d["V"] = d["K8"], d["V8"]
    g = torch.Generator(device=DEV).manual_seed(seed + 77)
    d["q"] = torch.randn((B, T, h, d_h), generator=g, device=DEV).to(torch.bfloat16)
    return sh, d


def host_kv(d):
    return synth.host_bits(d["K"]), synth.host_bits(d["V"])


def run(B, T, h, h_kv, d_h, s, seed, paged=False, fp8=None):
    print(f"[multi] B={B} q_len={T} h={h} h_kv={h_kv} d_h={d_h} s={list(s)[:6]} paged={paged} "
          f"fp8={fp8 is not None}", flush=True)
    sh, d = draw(B, T, h, h_kv, d_h, s, seed, paged, fp8)
    ks, vs = (None, None) if fp8 is None else fp8
    out, lse = A.decode_gqa_multi(d["q"], d["K"], d["V"], d["s"], block_table=d.get("block_table"),
                                  s_max=sh.s_max, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    hK, hV = host_kv(d)
    kw = dict(block_table=d.get("block_table_host"))
    if fp8 is None:
        ref, ref_lse = oracle.gqa_decode_multi(synth.host_bits(d["q"]), hK, hV, d["s_host"], 2, **kw)
    else:
        ref, ref_lse = oracle.gqa_decode_multi(synth.host_bits(d["q"]), hK, hV, d["s_host"], 1,
                                               k_scale=ks, v_scale=vs, **kw)
    assert_close(to_f64(out), ref, 2, "out")
    assert_lse_close(to_f64(lse), ref_lse, 2, "lse")
    return sh, d, out, lse


@pytest.mark.parametrize("T", [2, 3, 4, 8])
@pytest.mark.parametrize("h,h_kv", [(32, 8), (8, 8), (64, 8), (16, 1)])
@pytest.mark.parametrize("d_h", [64, 128])
def test_positions_and_group_sizes(T, h, h_kv, d_h):
    run(3, T, h, h_kv, d_h, (1, 77, 300), seed=T * 100 + h + h_kv)


@pytest.mark.parametrize("T,h,h_kv", [(2, 64, 1), (8, 16, 1), (64, 8, 8), (5, 40, 2), (16, 128, 1)])
def test_row_blocks_beyond_64(T, h, h_kv):
    # g * q_len rows above 64 run as several 64-row workgroups per KV head
    run(2, T, h, h_kv, 128, (200, 33), seed=T * 7 + h)


@pytest.mark.parametrize("s", [(0, 1), (2, 3), (4, 5), (31, 33)])
def test_sequences_shorter_than_or_near_q_len(s):
    run(2, 4, 16, 4, 128, s, seed=sum(s) + 3)


def test_split_context():
    run(1, 4, 32, 8, 128, (9000,), seed=21)
    run(2, 8, 16, 2, 128, (5000, 4), seed=22)


def test_split_boundary_leaves_early_positions_empty():
    # the last split holds only the newest tokens: earlier positions see none of it
    run(1, 8, 16, 2, 128, (4097,), seed=23)
    run(1, 8, 16, 2, 128, (4100,), seed=24)


@pytest.mark.parametrize("T", [2, 5])
def test_paged_shuffled(T):
    run(4, T, 32, 8, 128, (1, 16, 17, 500), seed=25 + T, paged=True)


@pytest.mark.parametrize("T", [2, 4])
def test_fp8_caches(T):
    run(3, T, 32, 8, 128, (5, 300, 1000), seed=30 + T, fp8=(1 / 64, 1 / 32))
    run(2, T, 16, 4, 64, (2, 700), seed=40 + T, fp8=(0.02, 0.05), paged=True)


def test_one_position_equals_single_token_call():
    sh, d = draw(3, 1, 32, 8, 128, (5, 900, 4096), seed=50)
    o1, l1 = A.decode_gqa_multi(d["q"], d["K"], d["V"], d["s"])
    o2, l2 = A.decode_gqa(d["q"][:, 0].contiguous(), d["K"], d["V"], d["s"])
    torch.cuda.synchronize()
    assert torch.equal(o1[:, 0].view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1[:, 0], l2)


def sampled(name, T, fp8=None):
    sh0 = synth.configs()[name]
    print(f"[multi-full] {name} q_len={T} fp8={fp8 is not None}", flush=True)
    sh, d = draw(sh0.B, T, sh0.h, sh0.h_kv, sh0.d_h, sh0.s, sh0.seed, sh0.paged, fp8)
    ks, vs = (None, None) if fp8 is None else fp8
    out, lse = A.decode_gqa_multi(d["q"], d["K"], d["V"], d["s"], block_table=d.get("block_table"),
                                  s_max=sh.s_max, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    g = sh.h // sh.h_kv
    rng = np.random.default_rng(1)
    for bi in sorted({0, sh.B - 1, int(rng.integers(0, sh.B))}):
        j = int(rng.integers(0, sh.h_kv))
        n = int(sh.s[bi])
        if sh.paged:
            tab = d["block_table_host"][bi]
            nb = (n + 15) // 16
            idx = torch.as_tensor(tab[:nb], dtype=torch.long, device=DEV)
            Kb = d["K"].index_select(0, idx).reshape(-1, sh.h_kv, sh.d_h)[:n, j]
            Vb = d["V"].index_select(0, idx).reshape(-1, sh.h_kv, sh.d_h)[:n, j]
        else:
            Kb, Vb = d["K"][bi, :n, j], d["V"][bi, :n, j]
        q = synth.host_bits(d["q"][bi:bi + 1, :, j * g:(j + 1) * g].contiguous())
        K = synth.host_bits(Kb.contiguous())[None, :, None, :]
        V = synth.host_bits(Vb.contiguous())[None, :, None, :]
        b = 2 if fp8 is None else 1
        ro, rl = oracle.gqa_decode_multi(q, K, V, np.array([n], np.int32), b,
                                         k_scale=ks or 1.0, v_scale=vs or 1.0)
        assert_close(to_f64(out[bi:bi + 1, :, j * g:(j + 1) * g]), ro, 2, f"{name} b={bi} j={j}")
        assert_lse_close(to_f64(lse[bi:bi + 1, :, j * g:(j + 1) * g]), rl, 2, f"{name} b={bi} j={j}")


@pytest.mark.parametrize("name", ["llama3_8b_gqa", "llama3_70b_gqa8_b16", "llama3_70b_mqa_b1",
                                  "paged_gqa8"])
def test_full_size_four_drafted_tokens_sampled(name):
    sampled(name, 4)


def test_full_size_fp8_sampled():
    sampled("llama3_70b_gqa8_b16", 4, fp8=(1 / 64, 1 / 64))


def test_bad_arguments():
    sh, d = draw(1, 2, 8, 2, 128, (10,), seed=60)
    out = torch.empty_like(d["q"])
    for q_len, b, code in ((0, 2, A.ATTN_EINVAL), (65, 2, A.ATTN_EINVAL), (2, 4, A.ATTN_ENOTSUP),
                           (2, 1, A.ATTN_ENOTSUP)):
        rc = A.attn_decode_gqa_multi(out, None, d["q"], d["K"], d["V"], d["s"], None, 0, 16, 0, 1,
                                     q_len, sh.s_max, 8, 2, 128, b, 0.0, None, 0, check=False)
        assert rc == code, (q_len, b, rc, A.attn_last_error())
    assert A.attn_decode_gqa_multi_workspace_bytes(1, 0, 10, 8, 2, 128) == 0


def test_paged_mixed_lengths_many_splits():
    s = (0, 5000, 2, 700, 0, 9000, 33, 4096, 4097, 3)
    run(10, 4, 32, 8, 128, s, seed=70, paged=True)
    run(10, 2, 16, 4, 128, s, seed=71, paged=True, fp8=(1 / 64, 1 / 32))
