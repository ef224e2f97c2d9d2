"""GPU parity of GQA/MQA/MHA decode over batches of mixed lengths.

Batches with many (sequence, KV head) pairs, mixed and empty lengths, one
long context among many empty or one-token ones, paged pools, E4M3 caches
(per-tensor and per-page scales), several new tokens per sequence (two row
blocks per KV head), and calls of different shapes sharing one workspace,
all against the oracle, with either form of the split merge.
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


@pytest.fixture(autouse=True, params=["kernel", "fused"])
def merge_form(request, monkeypatch):
    """Every test runs with both forms of the split merge: the separate merge
    kernel (default) and the merge by the last workgroup of each item inside
    the decode kernel (ATTN_GQA_MERGE=fused)."""
    if request.param == "fused":
        monkeypatch.setenv("ATTN_GQA_MERGE", "fused")
    else:
        monkeypatch.delenv("ATTN_GQA_MERGE", raising=False)
    print(f"[merge={request.param}]", flush=True)
    return request.param


def lengths(B, seed, lo=0, hi=3000, zeros=()):
    rng = np.random.default_rng(seed)
    s = rng.integers(lo, hi + 1, size=B)
    for i in zeros:
        s[i] = 0
    return tuple(int(x) for x in s)


def check_gqa(sh, d, out, lse, what):
    ref, ref_lse = oracle.gqa_decode(*(synth.host_bits(d[k]) for k in ("q", "K", "V")), d["s_host"],
                                     sh.b, block_table=d.get("block_table_host"))
    assert_close(to_f64(out), ref, sh.b, what)
    assert_lse_close(to_f64(lse), ref_lse, sh.b, what)


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("h,h_kv,d_h", [(16, 2, 128), (8, 1, 128), (64, 2, 64)])
def test_mixed_lengths_fused_merge(paged, h, h_kv, d_h):
    B = 64 if h_kv == 1 else 40
    s = lengths(B, seed=h + h_kv + d_h, hi=4000, zeros=(0, 7))
    s = s[:3] + (1, 31, 33) + s[6:]
    print(f"[gqa-mixed] B={B} h={h} h_kv={h_kv} d_h={d_h} paged={paged}", flush=True)
    sh = synth.GqaShape("t", B=B, h=h, h_kv=h_kv, d_h=d_h, b=2, s=s, paged=paged, seed=900 + h)
    d = synth.draw_gqa(sh, device=DEV)
    out, lse = A.decode_gqa(d["q"], d["K"], d["V"], d["s"], block_table=d.get("block_table"),
                            s_max=sh.s_max)
    torch.cuda.synchronize()
    check_gqa(sh, d, out, lse, "out")


def test_one_long_context_among_empty_and_single_token_ones():
    # 63 empty or one-token sequences and one of 140,000 tokens over one KV
    # head: the long context is split many ways, the others not at all
    s = tuple([0, 1] * 31 + [0]) + (140000,)
    print("[gqa-mixed] one long segment, 63 short ones", flush=True)
    sh = synth.GqaShape("t", B=64, h=8, h_kv=1, d_h=128, b=2, s=s, seed=911)
    d = synth.draw_gqa(sh, device=DEV)
    out, lse = A.decode_gqa(d["q"], d["K"], d["V"], d["s"])
    torch.cuda.synchronize()
    check_gqa(sh, d, out, lse, "out")
    o = to_f64(out)
    assert np.all(o[0::2][:32] == 0.0) and np.all(np.isneginf(to_f64(lse)[0:62:2]))


def test_repeated_calls_share_one_workspace():
    # the same workspace gives the same bits on a repeat, and serves calls of
    # other shapes in between
    ws = A.Workspace(DEV)
    sh1 = synth.GqaShape("t", B=48, h=32, h_kv=4, d_h=128, b=2, s=lengths(48, 3, hi=5000), seed=921)
    sh2 = synth.GqaShape("t", B=70, h=8, h_kv=1, d_h=64, b=2, s=lengths(70, 4, hi=2500), paged=True,
                         seed=922)
    d1 = synth.draw_gqa(sh1, device=DEV)
    d2 = synth.draw_gqa(sh2, device=DEV)
    print("[gqa-mixed] repeated calls on one workspace", flush=True)
    o1, l1 = A.decode_gqa(d1["q"], d1["K"], d1["V"], d1["s"], workspace=ws)
    o2, l2 = A.decode_gqa(d2["q"], d2["K"], d2["V"], d2["s"], block_table=d2["block_table"],
                          s_max=sh2.s_max, workspace=ws)
    o3, l3 = A.decode_gqa(d1["q"], d1["K"], d1["V"], d1["s"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16)) and torch.equal(l1, l3)
    check_gqa(sh1, d1, o1, l1, "first shape")
    check_gqa(sh2, d2, o2, l2, "second shape")


@pytest.mark.parametrize("paged", [False, True])
def test_fp8_per_tensor_scales(paged):
    ks, vs = 1.0 / 64, 0.0123
    s = lengths(64, 5, hi=3000, zeros=(3,))
    sh = synth.GqaShape("t", B=64, h=16, h_kv=2, d_h=128, b=2, s=s, paged=paged, seed=931)
    print(f"[gqa-mixed] fp8 paged={paged}", flush=True)
    d = synth.draw_gqa_fp8(sh, ks, vs, device=DEV)
    out, lse = A.decode_gqa_fp8(d["q"], d["K8"], d["V8"], ks, vs, d["s"],
                                block_table=d.get("block_table"), s_max=sh.s_max)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.gqa_decode_fp8(synth.host_bits(d["q"]), synth.host_bits(d["K8"]),
                                         synth.host_bits(d["V8"]), ks, vs, d["s_host"],
                                         block_table=d.get("block_table_host"))
    assert_close(to_f64(out), ref, 2, "out")
    assert_lse_close(to_f64(lse), ref_lse, 2, "lse")


def test_fp8_per_page_scales():
    from tests.test_gpu_fp8 import page_scaled_pool
    B, h, h_kv, d_h = 40, 16, 2, 128
    s = lengths(B, 6, hi=4000, zeros=(1,))
    sh = synth.GqaShape("t", B=B, h=h, h_kv=h_kv, d_h=d_h, b=2, s=s, paged=True, seed=941)
    print("[gqa-mixed] fp8 per-page scales", flush=True)
    d, K8, V8, ksc, vsc = page_scaled_pool(sh, seed=941)
    bt = d["block_table"]
    out = torch.empty_like(d["q"])
    lse = torch.empty((B, h), dtype=torch.float32, device=DEV)
    wsb = A.attn_decode_workspace_bytes(0, B, sh.s_max, h, h_kv, d_h)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=DEV)
    A.attn_decode_gqa_fp8_paged_scales(out, lse, d["q"], K8, V8, ksc, vsc, d["s"], bt, bt.shape[1],
                                       16, K8.shape[0], B, sh.s_max, h, h_kv, d_h, 0.0, ws, wsb)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.gqa_decode_fp8_paged_scales(synth.host_bits(d["q"]), synth.host_bits(K8),
                                                      synth.host_bits(V8), ksc.cpu().numpy(),
                                                      vsc.cpu().numpy(), d["s_host"],
                                                      d["block_table_host"])
    assert_close(to_f64(out), ref, 2, "out")
    assert_lse_close(to_f64(lse), ref_lse, 2, "lse")


@pytest.mark.parametrize("paged", [False, True])
def test_several_new_tokens_two_row_blocks(paged):
    # g = 32 query heads per KV head and 8 new tokens: 256 rows per KV head,
    # two row blocks of 128; 16 sequences x 2 KV heads x 2 blocks = 64 segments
    B, q_len, h, h_kv, d_h = 16, 8, 64, 2, 128
    s = lengths(B, 7, lo=3, hi=3000)
    s = (5, 8) + s[2:]
    sh = synth.GqaShape("t", B=B, h=h, h_kv=h_kv, d_h=d_h, b=2, s=s, paged=paged, seed=951)
    print(f"[gqa-mixed] q_len={q_len} paged={paged}", flush=True)
    d = synth.draw_gqa(sh, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(952)
    q = torch.randn((B, q_len, h, d_h), generator=g, device=DEV).to(torch.bfloat16)
    out, lse = A.decode_gqa_multi(q, d["K"], d["V"], d["s"], block_table=d.get("block_table"),
                                  s_max=sh.s_max)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.gqa_decode_multi(synth.host_bits(q), synth.host_bits(d["K"]),
                                           synth.host_bits(d["V"]), d["s_host"], 2,
                                           block_table=d.get("block_table_host"))
    assert_close(to_f64(out), ref, 2, "out")
    assert_lse_close(to_f64(lse), ref_lse, 2, "lse")


def _gqa_call(sh, d, ws, wsb):
    bt = d.get("block_table")
    mb = 0 if bt is None else bt.shape[1]
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full((sh.B, sh.h), float("nan"), dtype=torch.float32, device=DEV)
    rc = A.attn_decode_gqa(out, lse, d["q"], d["K"], d["V"], d["s"], bt, mb, sh.block_size,
                           0 if bt is None else d["K"].shape[0], sh.B, sh.s_max, sh.h, sh.h_kv,
                           sh.d_h, sh.b, 0.0, ws, wsb)
    assert rc == A.ATTN_OK
    return out, lse


@pytest.mark.parametrize("paged", [False, True])
def test_many_splits_and_empty_sequences_counters_left_zero(paged):
    # one item with about 270 splits, one with a few, empty and one-token
    # sequences (one workgroup each, nothing to merge); with the in-kernel
    # merge the last workgroup of each item merges its splits, and every
    # call leaves the workspace's arrival counters at zero, so a second call
    # on the same workspace gives the same bits
    s = (0, 140000, 1, 0, 9000, 5)
    sh = synth.GqaShape("t", B=len(s), h=16, h_kv=1, d_h=128, b=2, s=s, paged=paged, seed=961)
    print(f"[gqa-fused] paged={paged}", flush=True)
    d = synth.draw_gqa(sh, device=DEV)
    wsb = A.attn_decode_workspace_bytes(0, sh.B, sh.s_max, sh.h, sh.h_kv, sh.d_h)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    o1, l1 = _gqa_call(sh, d, ws, wsb)
    torch.cuda.synchronize()
    assert torch.all(ws[:65536] == 0), "arrival counters not left at zero"
    o2, l2 = _gqa_call(sh, d, ws, wsb)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    assert torch.all(ws[:65536] == 0)
    check_gqa(sh, d, o1, l1, "out")
    o = to_f64(o1)
    assert np.all(o[[0, 3]] == 0.0) and np.all(np.isneginf(to_f64(l1)[[0, 3]]))


def test_more_items_than_arrival_counters_use_the_merge_kernel():
    # 2,100 sequences x 8 KV heads = 16,800 (sequence, KV head) items with
    # two splits each: more than the 16,384 counters of the workspace
    # prefix, so the separate merge kernel combines the splits
    from tests._gpu import gqa_sample_reference
    B = 2100
    rng = np.random.default_rng(971)
    s = [int(x) for x in rng.integers(0, 200, size=B)]
    s[0], s[1], s[5], s[B - 1] = 8192, 0, 4097, 6000
    sh = synth.GqaShape("t", B=B, h=32, h_kv=8, d_h=128, b=2, s=tuple(s), paged=True, seed=971)
    print("[gqa-fused] 16,800 items, merge kernel", flush=True)
    d = synth.draw_gqa(sh, device=DEV)
    wsb = A.attn_decode_workspace_bytes(0, sh.B, sh.s_max, sh.h, sh.h_kv, sh.d_h)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    out, lse = _gqa_call(sh, d, ws, wsb)
    torch.cuda.synchronize()
    assert torch.all(ws[:65536] == 0)
    g = sh.h // sh.h_kv
    o64, l64 = to_f64(out), to_f64(lse)
    for (bi, j), (ro, rl) in gqa_sample_reference(d, sh, [(0, 0), (1, 3), (5, 7), (B - 1, 2), (700, 5)]).items():
        assert_close(o64[bi, j * g:(j + 1) * g], ro, 2, f"b={bi} j={j}")
        assert_lse_close(l64[bi, j * g:(j + 1) * g], rl, 2, f"b={bi} j={j}")
