"""GPU parity of attn_merge_partials against the oracle's merge, and of the
context-parallel path it serves: decode over token slices of a cache (one
slice per would-be GPU), then merge, against the oracle's decode over the
whole cache.

Tolerances: fp32 output max-abs <= 1e-5 against the oracle merge of the same
partials; bf16 output the bf16 bar (max-abs <= 2e-2, mean-abs <= 2e-3,
rel-RMS <= 1e-2); lse as in the decode tests.
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


def random_parts(n, B, h, d, dtype, seed, empty_frac=0.2):
    g = torch.Generator(device="cpu").manual_seed(seed)
    o = torch.randn((n, B, h, d), generator=g).to(dtype)
    lse = (torch.randn((n, B, h), generator=g) * 4.0).float()
    lse[torch.rand((n, B, h), generator=g) < empty_frac] = -float("inf")
    return o.to(DEV), lse.to(DEV)


def host_parts(o, lse):
    return synth.host_bits(o), lse.cpu().numpy()


@pytest.mark.parametrize("n", [1, 3, 8, 13, 70])
@pytest.mark.parametrize("d", [64, 128, 512, 576, 1024])
@pytest.mark.parametrize("io", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"), ("bf16", "f32")])
def test_merge_matches_oracle(n, d, io):
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}
    B, h = 3, 5
    print(f"[merge] n={n} d={d} io={io}", flush=True)
    o, l = random_parts(n, B, h, d, dt[io[0]], seed=n * 1000 + d)
    out, lse = A.merge_partials(o, l, out_dtype=dt[io[1]])
    torch.cuda.synchronize()
    ho, hl = host_parts(o, l)
    ref, ref_lse = oracle.merge_partials(ho, hl, 2 if io[0] == "bf16" else 4)
    if io[1] == "f32":
        assert np.max(np.abs(to_f64(out) - ref)) <= 1e-5
    else:
        # only the final rounding to bf16 differs: half an ulp of |ref|
        err = np.abs(to_f64(out) - ref)
        assert np.all(err <= np.abs(ref) * 2.0 ** -8 + 1e-6)
    assert_lse_close(to_f64(lse), ref_lse, 4, "lse")


def test_single_slice_is_bitwise_identity():
    for dt in (torch.float32, torch.bfloat16):
        o, l = random_parts(1, 4, 8, 128, dt, seed=5, empty_frac=0.0)
        out, lse = A.merge_partials(o, l)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8), o[0].contiguous().view(torch.uint8))
        assert torch.equal(lse, l[0])


def test_all_slices_empty_gives_zero_and_neg_inf():
    o, l = random_parts(4, 2, 3, 128, torch.bfloat16, seed=6)
    l[:, 1, 2] = -float("inf")
    l[:, 0, :] = -float("inf")
    out, lse = A.merge_partials(o, l)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0) and torch.all(out[1, 2] == 0)
    assert torch.all(torch.isneginf(lse[0])) and torch.isneginf(lse[1, 2])
    assert torch.all(torch.isfinite(lse[1, :2]))


def test_empty_slice_rows_are_not_read():
    # an empty slice's out row holds NaN here: the merge must not read it into the sum
    o, l = random_parts(5, 2, 4, 128, torch.float32, seed=7, empty_frac=0.0)
    l[2] = -float("inf")
    o[2] = float("nan")
    out, lse = A.merge_partials(o, l)
    ref, ref_l = A.merge_partials(o[[0, 1, 3, 4]].contiguous(), l[[0, 1, 3, 4]].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(lse, ref_l)


def slices(x, n, s_max):
    """Token-axis slices [:, kS:(k+1)S] of a contiguous cache, S = ceil(s_max / n)."""
    S = (s_max + n - 1) // n
    return S, [x[:, k * S:min((k + 1) * S, s_max)].contiguous() for k in range(n)]


def local_lengths(s, k, S):
    return torch.clamp(s - k * S, min=0, max=S).to(torch.int32)


def dcp_gqa(d, sh, n):
    S, Ks = slices(d["K"], n, sh.s_max)
    _, Vs = slices(d["V"], n, sh.s_max)
    outs, lses = [], []
    for k in range(n):
        sk = local_lengths(d["s"], k, S)
        o, l = A.decode_gqa(d["q"], Ks[k], Vs[k], sk, s_max=Ks[k].shape[1])
        outs.append(o)
        lses.append(l)
    return A.merge_partials(torch.stack(outs), torch.stack(lses))


@pytest.mark.parametrize("n", [2, 4, 7])
def test_context_parallel_gqa_equals_whole_decode(n):
    sh = synth.GqaShape("t", B=3, h=16, h_kv=2, d_h=128, b=2, s=(3000, 700, 1), seed=41)
    print(f"[merge-dcp-gqa] n={n}", flush=True)
    d = synth.draw_gqa(sh, device=DEV)
    out, lse = dcp_gqa(d, sh, n)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.gqa_decode(*(synth.host_bits(d[k]) for k in ("q", "K", "V")),
                                     d["s_host"], 2)
    assert_close(to_f64(out), ref, 2, "out")
    assert_lse_close(to_f64(lse), ref_lse, 2, "lse")


def test_context_parallel_gqa_fp32_slices():
    sh = synth.GqaShape("t", B=2, h=8, h_kv=2, d_h=64, b=4, s=(900, 37), seed=42)
    d = synth.draw_gqa(sh, device=DEV)
    out, lse = dcp_gqa(d, sh, 3)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.gqa_decode(*(synth.host_bits(d[k]) for k in ("q", "K", "V")),
                                     d["s_host"], 4)
    assert_close(to_f64(out), ref, 4, "out")
    assert_lse_close(to_f64(lse), ref_lse, 4, "lse")


def test_context_parallel_70b_gqa8_b1_eight_slices_sampled():
    # Llama-3-70B GQA-8 at B=1, s=131072, cut into 8 slices of 16384 tokens
    sh = synth.configs()["llama3_70b_gqa8_b1"]
    print(f"[merge-dcp-gqa] {sh.name} n=8", flush=True)
    d = synth.draw_gqa(sh, device=DEV)
    out, lse = dcp_gqa(d, sh, 8)
    torch.cuda.synchronize()
    g = sh.h // sh.h_kv
    pairs = [(0, 0), (0, 5), (0, sh.h_kv - 1)]
    ref = gqa_sample_reference(d, sh, pairs)
    o64, l64 = to_f64(out), to_f64(lse)
    for (bi, j), (ro, rl) in ref.items():
        assert_close(o64[bi, j * g:(j + 1) * g], ro, 2, f"j={j}")
        assert_lse_close(l64[bi, j * g:(j + 1) * g], rl, 2, f"j={j}")


def test_context_parallel_mla_equals_whole_decode():
    sh = synth.MlaShape("t", B=3, h=32, d_c=512, d_R=64, d_nope=128, d_v=128, s=(2000, 300, 0),
                        seed=43)
    print("[merge-dcp-mla] n=3", flush=True)
    d = synth.draw_mla(sh, device=DEV)
    n = 3
    S, Cs = slices(d["cache"], n, sh.s_max)
    outs, lats, lses = [], [], []
    for k in range(n):
        sk = local_lengths(d["s"], k, S)
        o, u, l = A.decode_mla(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], Cs[k], sk,
                               s_max=Cs[k].shape[1])
        outs.append(o)
        lats.append(u)
        lses.append(l)
    out, lse = A.merge_partials(torch.stack(outs), torch.stack(lses))
    lat, _ = A.merge_partials(torch.stack(lats), torch.stack(lses))
    torch.cuda.synchronize()
    ro, ru, rl = oracle.mla_absorbed(*(synth.host_bits(d[k]) for k in
                                       ("q_nope", "q_rope", "w_uk", "w_uv", "cache")),
                                     d["s_host"])
    assert_close(to_f64(out), ro, 2, "out")
    assert_close(to_f64(lat), ru, 2, "u_latent")
    assert_lse_close(to_f64(lse), rl, 2, "lse")


def test_bad_arguments():
    o, l = random_parts(2, 1, 2, 128, torch.bfloat16, seed=8)
    out = torch.empty((1, 2, 128), dtype=torch.bfloat16, device=DEV)
    cases = [
        (dict(n_parts=0), A.ATTN_EINVAL),
        (dict(h=0), A.ATTN_EINVAL),
        (dict(d=6), A.ATTN_ENOTSUP),
        (dict(d=1028), A.ATTN_ENOTSUP),
        (dict(b_parts=3), A.ATTN_ENOTSUP),
        (dict(o_parts=o.data_ptr() + 2), A.ATTN_EINVAL),
        (dict(o_parts=None), A.ATTN_EINVAL),
    ]
    for over, code in cases:
        kw = dict(out=out, lse=None, o_parts=o, lse_parts=l, n_parts=2, B=1, h=2, d=128,
                  b_parts=2, b_out=2)
        kw.update(over)
        rc = A.attn_merge_partials(**kw, check=False)
        assert rc == code, (over, rc, A.attn_last_error())
    # B = 0 is a valid empty call
    assert A.attn_merge_partials(out, None, o, l, 2, 0, 2, 128, 2, 2) == 0
