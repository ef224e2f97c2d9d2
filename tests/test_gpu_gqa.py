"""GPU parity of attn_decode_gqa (MHA / MQA / GQA) against the CPU oracle.

Small cases compare every output element; the full-size workloads
(Llama-3-8B and Llama-3-70B shaped layers, the paged mixed-length batch)
are run in the same launch configuration as the benchmark and compared on
sampled KV-head groups, which the oracle computes one by one.
Tolerances: bf16 storage max-abs <= 2e-2, mean-abs <= 2e-3 (plus rel-RMS
<= 1e-2); fp32 storage max-abs <= 1e-5.
"""
import numpy as np
import pytest
import torch

import decode_attention_kv_attn_amd as A
import oracle
import synth
from tests._gpu import assert_close, assert_lse_close, gqa_sample_reference, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_small(B, h, h_kv, d_h, s, b, seed, paged=False, block_table=None):
    sh = synth.GqaShape("t", B=B, h=h, h_kv=h_kv, d_h=d_h, b=b, s=tuple(s), paged=paged, seed=seed)
    print(f"[gqa] B={B} h={h} h_kv={h_kv} d_h={d_h} b={b} s={list(s)[:6]} paged={paged}", flush=True)
    d = synth.draw_gqa(sh, device=DEV)
    bt = d.get("block_table")
    out, lse = A.decode_gqa(d["q"], d["K"], d["V"], d["s"], block_table=bt, s_max=sh.s_max)
    torch.cuda.synchronize()
    hq, hK, hV = (synth.host_bits(d[k]) for k in ("q", "K", "V"))
    ref, ref_lse = oracle.gqa_decode(hq, hK, hV, d["s_host"], b,
                                     block_table=d.get("block_table_host"))
    assert_close(to_f64(out), ref, b, "out")
    assert_lse_close(to_f64(lse), ref_lse, b, "lse")
    return d, out, lse


def test_tiny_fp32_workload():
    # B=2, h=8, h_kv=2, d_h=64, s=[100, 256], fp32
    c = synth.configs()["tiny_gqa_fp32"]
    run_small(c.B, c.h, c.h_kv, c.d_h, c.s, c.b, c.seed)


@pytest.mark.parametrize("s", [(100,), (256,)])
def test_tiny_fp32_uniform_lengths(s):
    run_small(2, 8, 2, 64, s * 2, 4, seed=1)


# g = 1 .. 64 run on the matrix-core kernel (one to four wavefronts of 16
# heads, the last one possibly partial or idle); g = 96 and 128 take the
# vector kernel
@pytest.mark.parametrize("h,h_kv", [(8, 8), (8, 4), (16, 4), (32, 8), (16, 2), (64, 1), (12, 4), (6, 2),
                                    (40, 2), (48, 1), (96, 1), (128, 1)])
@pytest.mark.parametrize("d_h", [64, 128])
def test_bf16_group_sizes(h, h_kv, d_h):
    run_small(3, h, h_kv, d_h, (1, 77, 300), 2, seed=h * 100 + h_kv)


@pytest.mark.parametrize("s", [(0, 5), (0, 0), (1, 1), (31, 33), (32, 64), (63, 65)])
def test_bf16_ragged_and_degenerate(s):
    run_small(2, 8, 2, 128, s, 2, seed=7)


def test_fp32_ragged_tail_and_empty():
    run_small(3, 8, 2, 64, (0, 1, 97), 4, seed=8)


@pytest.mark.parametrize("merge", ["kernel", "fused"])
def test_split_kv_long_context_small_batch(merge, monkeypatch):
    if merge == "fused":
        monkeypatch.setenv("ATTN_GQA_MERGE", "fused")
    # B=1 with a long context forces several splits plus the merge kernel
    run_small(1, 16, 2, 128, (20000,), 2, seed=9)
    run_small(2, 8, 1, 128, (9000, 3), 2, seed=10)
    run_small(1, 8, 2, 64, (5000,), 4, seed=11)


@pytest.mark.parametrize("merge", ["kernel", "fused"])
def test_split_kv_more_than_256_splits(merge, monkeypatch):
    if merge == "fused":
        monkeypatch.setenv("ATTN_GQA_MERGE", "fused")
    # one KV head over 140,000 tokens: about 270 splits of 512 tokens, merged
    # by the 16-wavefront form of the merge kernel, or by the item's last
    # workgroup
    run_small(1, 16, 1, 128, (140000,), 2, seed=12)


@pytest.mark.parametrize("b", [2, 4])
def test_paged_shuffled_table(b):
    run_small(4, 8, 2, 64, (1, 16, 17, 500), b, seed=12, paged=True)


def test_paged_bit_identical_to_identity_table():
    s = (5, 40, 129, 700)
    sh = synth.GqaShape("t", B=4, h=16, h_kv=4, d_h=128, b=2, s=s, paged=True, seed=13)
    d = synth.draw_gqa(sh, device=DEV)
    tab = d["block_table_host"]
    # same logical cache, stored in order: physical block = identity numbering
    ident, n_blk = synth.identity_table(s, 16)
    Kp, Vp = d["K"], d["V"]
    perm = torch.as_tensor(tab[tab >= 0], dtype=torch.long, device=DEV)
    order = torch.as_tensor(np.concatenate([tab[i, :(n + 15) // 16] for i, n in enumerate(s)]),
                            dtype=torch.long, device=DEV)
    Ki, Vi = Kp.index_select(0, order), Vp.index_select(0, order)
    o1, l1 = A.decode_gqa(d["q"], Kp, Vp, d["s"], block_table=d["block_table"], s_max=max(s))
    o2, l2 = A.decode_gqa(d["q"], Ki, Vi, d["s"], block_table=torch.from_numpy(ident).to(DEV),
                          s_max=max(s))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    del perm


def test_deterministic_repeat():
    sh = synth.GqaShape("t", B=2, h=32, h_kv=8, d_h=128, b=2, s=(3000, 4096), seed=14)
    d = synth.draw_gqa(sh, device=DEV)
    o1, l1 = A.decode_gqa(d["q"], d["K"], d["V"], d["s"])
    o2, l2 = A.decode_gqa(d["q"], d["K"], d["V"], d["s"])
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


FULL = ["llama3_8b_gqa", "llama3_70b_mha_b16", "llama3_70b_gqa8_b16", "llama3_70b_mqa_b16",
        "llama3_70b_mha_b1", "llama3_70b_gqa8_b1", "llama3_70b_mqa_b1", "paged_gqa8"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    sh = synth.configs()[name]
    print(f"[gqa-full] {name}", flush=True)
    d = synth.draw_gqa(sh, device=DEV)
    out, lse = A.decode_gqa(d["q"], d["K"], d["V"], d["s"], block_table=d.get("block_table"),
                            s_max=sh.s_max)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    nb = min(sh.B, 3)
    bs = sorted(set([0, sh.B - 1] + list(rng.integers(0, sh.B, size=nb))))
    pairs = [(int(bi), int(rng.integers(0, sh.h_kv))) for bi in bs]
    ref = gqa_sample_reference(d, sh, pairs)
    g = sh.h // sh.h_kv
    o64, l64 = to_f64(out), to_f64(lse)
    for (bi, j), (ro, rl) in ref.items():
        assert_close(o64[bi, j * g:(j + 1) * g], ro, sh.b, f"{name} b={bi} j={j}")
        assert_lse_close(l64[bi, j * g:(j + 1) * g], rl, sh.b, f"{name} b={bi} j={j}")
    assert np.all(np.isfinite(o64))


def test_peaked_logits_rescale():
    # a late key aligned with q makes the running max jump by a large amount
    sh = synth.GqaShape("t", B=2, h=16, h_kv=2, d_h=128, b=2, s=(700, 5000), seed=15)
    d = synth.draw_gqa(sh, device=DEV)
    for bi, t in ((0, 650), (1, 4500)):
        q0 = d["q"][bi, 0].float()
        d["K"][bi, t, 0] = (q0 / q0.norm() * 60.0).to(torch.bfloat16)
    out, lse = A.decode_gqa(d["q"], d["K"], d["V"], d["s"])
    torch.cuda.synchronize()
    ref, ref_lse = oracle.gqa_decode(*(synth.host_bits(d[k]) for k in ("q", "K", "V")),
                                     d["s_host"], 2)
    assert ref_lse[0, 0] > 20
    assert_close(to_f64(out), ref, 2, "out")
    assert_lse_close(to_f64(lse), ref_lse, 2, "lse")


@pytest.mark.parametrize("merge", ["kernel", "fused"])
def test_paged_mixed_lengths_many_splits(merge, monkeypatch):
    if merge == "fused":
        monkeypatch.setenv("ATTN_GQA_MERGE", "fused")
    # empty sequences, one-token ones and several splits per sequence in one
    # paged batch: the workgroups map onto the non-empty (sequence, split)
    # pairs only, and the merge reads only the splits each sequence has
    s = (0, 5000, 1, 700, 0, 9000, 33, 4096, 4097, 0, 12000, 64)
    run_small(12, 16, 2, 128, s, 2, seed=16, paged=True)
    run_small(12, 8, 8, 64, s, 2, seed=17, paged=True)


@pytest.mark.parametrize("paged", [False, True])
def test_large_batch_short_sequences(paged):
    # more sequences than the compacted split mapping scans (B > 1024), with
    # empty and one-token ones among them; sampled rows against the oracle
    B = 1500
    rng = np.random.default_rng(18)
    s = tuple(int(x) for x in rng.integers(0, 300, size=B))
    s = (0, 1) + s[2:]
    sh = synth.GqaShape("t", B=B, h=32, h_kv=8, d_h=128, b=2, s=s, paged=paged, seed=18)
    print(f"[gqa-largeB] paged={paged}", flush=True)
    d = synth.draw_gqa(sh, device=DEV)
    out, lse = A.decode_gqa(d["q"], d["K"], d["V"], d["s"], block_table=d.get("block_table"),
                            s_max=sh.s_max)
    torch.cuda.synchronize()
    pairs = [(0, 0), (1, 3), (2, 7), (700, 2), (B - 1, 5)]
    ref = gqa_sample_reference(d, sh, pairs)
    g = sh.h // sh.h_kv
    o64, l64 = to_f64(out), to_f64(lse)
    for (bi, j), (ro, rl) in ref.items():
        assert_close(o64[bi, j * g:(j + 1) * g], ro, 2, f"b={bi} j={j}")
        assert_lse_close(l64[bi, j * g:(j + 1) * g], rl, 2, f"b={bi} j={j}")
    assert np.all(np.isfinite(o64))


def at_offset(x, offset):
    # a copy of x whose storage starts `offset` bytes past a fresh allocation
    nb = x.numel() * x.element_size()
    flat = torch.empty(nb + offset, dtype=torch.uint8, device=DEV)
    v = flat[offset:offset + nb].view(x.dtype).view(x.shape)
    v.copy_(x)
    return v


@pytest.mark.parametrize("offset", [0, 128, 256, 768])
@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("h,h_kv,d_h", [(32, 8, 128), (16, 4, 64), (64, 64, 128)])
def test_cache_alignment_and_head_order(offset, fp8, h, h_kv, d_h):
    # contiguous caches on the matrix cores take their KV heads in an order
    # set by bit 8 of the cache's address (plain order when it is not
    # 256-byte aligned): every alignment gives the oracle's results
    print(f"[gqa-align] offset={offset} fp8={fp8} h={h} h_kv={h_kv} d_h={d_h}", flush=True)
    sh = synth.GqaShape("t", B=3, h=h, h_kv=h_kv, d_h=d_h, b=2, s=(5, 700, 4500), seed=800 + offset + h)
    if fp8:
        ks, vs = 1 / 64, 1 / 32
        d = synth.draw_gqa_fp8(sh, ks, vs, device=DEV)
        K, V = at_offset(d["K8"], offset), at_offset(d["V8"], offset)
        out, lse = A.decode_gqa_fp8(d["q"], K, V, ks, vs, d["s"])
        ref, ref_lse = oracle.gqa_decode_fp8(synth.host_bits(d["q"]), synth.host_bits(d["K8"]),
                                             synth.host_bits(d["V8"]), ks, vs, d["s_host"])
    else:
        d = synth.draw_gqa(sh, device=DEV)
        K, V = at_offset(d["K"], offset), at_offset(d["V"], offset)
        out, lse = A.decode_gqa(d["q"], K, V, d["s"])
        ref, ref_lse = oracle.gqa_decode(*(synth.host_bits(d[k]) for k in ("q", "K", "V")),
                                         d["s_host"], 2)
    torch.cuda.synchronize()
    assert_close(to_f64(out), ref, 2, "out")
    assert_lse_close(to_f64(lse), ref_lse, 2, "lse")
