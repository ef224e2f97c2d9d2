"""GPU parity of the MLA output path -- attn_decode_mla_out (deferred: heads'
outputs, then W_O) and attn_decode_mla_out_premerged (merged weight W_O^i
W_UV,i built by attn_mla_premerge_weights) -- against the oracle's
oracle.mla_output (pinned to torch attention on the explicit expansion
followed by W_O).

Tolerance: the bf16 bounds of the other MLA tests (max-abs <= 2e-2,
mean-abs <= 2e-3, rel-RMS <= 1e-2) on the projected output, whose entries
are O(0.1): the deferred form rounds the heads' outputs to bf16 before the
projection, the merged form rounds u~ and the merged weight to bf16; both
sum in fp32 and round the result to bf16.
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


def shape(B, h, s, q_len=1, paged=False, seed=31, d_nope=128, d_v=128, d_model=512):
    return synth.MlaShape("t", B=B, h=h, d_c=512, d_R=64, d_nope=d_nope, d_v=d_v, s=tuple(s),
                          paged=paged, seed=seed, q_len=q_len, d_model=d_model)


def rows_of(d, sh, bi):
    n = int(sh.s[bi])
    if sh.paged:
        tab = d["block_table_host"][bi]
        nb = (n + sh.block_size - 1) // sh.block_size
        idx = torch.as_tensor(tab[:nb], dtype=torch.long, device=DEV)
        return d["cache"].index_select(0, idx).reshape(-1, sh.d_c + sh.d_R)[:max(n, 1)]
    return d["cache"][bi, :max(n, 1)]


def run(sh, merged, sample=None):
    print(f"[mla-out] B={sh.B} q_len={sh.q_len} h={sh.h} d_v={sh.d_v} d_model={sh.d_model} "
          f"s={list(sh.s)[:6]} paged={sh.paged} merged={merged}", flush=True)
    d = synth.draw_mla(sh, device=DEV)
    w_o = synth.draw_w_o(sh, device=DEV)
    kw = dict(block_table=d.get("block_table"), s_max=sh.s_max)
    if merged:
        w_abs = A.premerge_weights(w_o, d["w_uv"])
        out, lse = A.decode_mla_out(d["q_nope"], d["q_rope"], d["w_uk"], None, d["cache"], d["s"],
                                    w_absorbed=w_abs, **kw)
    else:
        out, lse = A.decode_mla_out(d["q_nope"], d["q_rope"], d["w_uk"], w_o, d["cache"], d["s"],
                                    w_uv=d["w_uv"], **kw)
    torch.cuda.synchronize()
    W = [synth.host_bits(d["w_uk"]), synth.host_bits(d["w_uv"]), synth.host_bits(w_o)]
    for bi in (range(sh.B) if sample is None else sample):
        qn, qr = (synth.host_bits(d[k][bi:bi + 1]) for k in ("q_nope", "q_rope"))
        C = synth.host_bits(rows_of(d, sh, bi))[None]
        ro, rl = oracle.mla_output(qn, qr, *W, C, np.array([int(sh.s[bi])], np.int32))
        assert_close(to_f64(out[bi:bi + 1]), ro, 2, f"out b={bi}")
        assert_lse_close(to_f64(lse[bi:bi + 1]), rl, 2, f"lse b={bi}")
    return out, lse


@pytest.mark.parametrize("merged", [False, True])
@pytest.mark.parametrize("h", [16, 128])
def test_heads(merged, h):
    run(shape(3, h, (40, 700, 2049), seed=h + merged), merged)


@pytest.mark.parametrize("merged", [False, True])
def test_multi_token_and_ragged_rows(merged):
    # 5 sequences x 3 new tokens = 15 projection rows (one partial 32-row tile)
    run(shape(5, 32, (0, 2, 9, 300, 1500), q_len=3, seed=51 + merged), merged)


@pytest.mark.parametrize("merged", [False, True])
def test_more_than_32_rows_paged(merged):
    rng = np.random.default_rng(53)
    s = tuple(int(x) for x in rng.integers(1, 2000, size=40))
    run(shape(40, 16, s, paged=True, seed=53 + merged), merged, sample=[0, 17, 33, 39])


def test_single_k_split_small_projection():
    # h d_v = 16 x 32 = 512: four K steps, one workgroup per column block
    run(shape(2, 16, (100, 33), d_v=32, d_model=96, seed=55), False)


@pytest.mark.parametrize("merged", [False, True])
def test_deepseek_v3_full_size_sampled(merged):
    base = synth.configs()["deepseek_v3_mla"]
    sh = shape(base.B, base.h, base.s, seed=base.seed, d_model=5120)
    run(sh, merged, sample=[0, sh.B - 1])


def test_premerged_weight_against_float64_product():
    h, d_c, d_v, d_model = 4, 512, 128, 64
    g = torch.Generator(device=DEV).manual_seed(57)
    w_o = (torch.randn((d_model, h * d_v), generator=g, device=DEV) / 16).to(torch.bfloat16)
    w_uv = (torch.randn((h, d_v, d_c), generator=g, device=DEV) / 16).to(torch.bfloat16)
    w_abs = A.premerge_weights(w_o, w_uv)
    torch.cuda.synchronize()
    wo = w_o.double().cpu().reshape(d_model, h, d_v)
    ref = torch.stack([wo[:, i] @ w_uv[i].double().cpu() for i in range(h)], dim=1)
    ref = ref.reshape(d_model, h * d_c)
    got = w_abs.double().cpu()
    # bf16 rounding of an fp32 sum of d_v products
    assert torch.all((got - ref).abs() <= 2.0 ** -8 * ref.abs() + 1e-5)


def test_bad_arguments():
    sh = shape(1, 16, (40,), seed=59)
    d = synth.draw_mla(sh, device=DEV)
    w_o = torch.zeros((100, 16 * 128), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((1, 100), dtype=torch.bfloat16, device=DEV)
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device=DEV)
    rc = A.attn_decode_mla_out(out, None, d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], w_o,
                               d["cache"], d["s"], None, 0, 16, 0, 1, 1, 40, 16, 512, 64, 128,
                               128, 100, 2, 0.0, ws, ws.numel(), check=False)
    assert rc == A.ATTN_ENOTSUP                      # d_model not a multiple of 32
    need = A.attn_decode_mla_out_workspace_bytes(0, 1, 1, 16, 512, 64, 128, 128)
    rc = A.attn_decode_mla_out(out, None, d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], w_o,
                               d["cache"], d["s"], None, 0, 16, 0, 1, 1, 40, 16, 512, 64, 128,
                               128, 128, 2, 0.0, ws, need - 1, check=False)
    assert rc == A.ATTN_EWORKSPACE
