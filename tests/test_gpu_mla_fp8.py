"""GPU parity of attn_decode_mla_absorbed_fp8 (E4M3 latent cache with a
latent and a rotary scale) against the oracle's FP8 MLA decode, and of
kv_cache_append_mla_fp8 against the oracle's append (bit-exact).

Output and u_latent use the bf16 tolerances of the MLA tests (max-abs <=
2e-2, mean-abs <= 2e-3, rel-RMS <= 1e-2); the codes widen to bf16 exactly, the
scales ride on the bf16 absorbed query (rounded there) and on u~.
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
CS, RS = 1.0 / 32, 1.0 / 16


def shape(B, h, s, paged=False, seed=31, d_nope=128, d_v=128):
    return synth.MlaShape("t", B=B, h=h, d_c=512, d_R=64, d_nope=d_nope, d_v=d_v, s=tuple(s),
                          paged=paged, seed=seed)


def rows_of(d, sh, bi):
    n = int(sh.s[bi])
    if sh.paged:
        tab = d["block_table_host"][bi]
        nb = (n + sh.block_size - 1) // sh.block_size
        idx = torch.as_tensor(tab[:nb], dtype=torch.long, device=DEV)
        return d["cache8"].index_select(0, idx).reshape(-1, sh.d_c + sh.d_R)[:max(n, 1)]
    return d["cache8"][bi, :max(n, 1)]


def check(d, sh, out, ul, lse, cs, rs, sample=None):
    for bi in (range(sh.B) if sample is None else sample):
        n = int(sh.s[bi])
        args = [synth.host_bits(d[k][bi:bi + 1]) for k in ("q_nope", "q_rope")]
        ro, ru, rl = oracle.mla_absorbed_fp8(args[0], args[1], synth.host_bits(d["w_uk"]),
                                             synth.host_bits(d["w_uv"]),
                                             synth.host_bits(rows_of(d, sh, bi))[None], cs, rs,
                                             np.array([n], np.int32))
        assert_close(to_f64(out[bi:bi + 1]), ro, 2, f"out b={bi}")
        assert_close(to_f64(ul[bi:bi + 1]), ru, 2, f"u_latent b={bi}")
        assert_lse_close(to_f64(lse[bi:bi + 1]), rl, 2, f"lse b={bi}")


def run(sh, cs=CS, rs=RS, sample=None):
    print(f"[mla-fp8] {sh.name} B={sh.B} h={sh.h} s={list(sh.s)[:6]} paged={sh.paged} "
          f"scales={cs},{rs}", flush=True)
    d = synth.draw_mla_fp8(sh, cs, rs, device=DEV)
    out, ul, lse = A.decode_mla(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["cache8"], d["s"],
                                block_table=d.get("block_table"), s_max=sh.s_max,
                                c_scale=cs, r_scale=rs)
    torch.cuda.synchronize()
    check(d, sh, out, ul, lse, cs, rs, sample)
    return d, out, ul, lse


@pytest.mark.parametrize("h", [16, 32, 128])
def test_head_counts(h):
    run(shape(2, h, (77, 300), seed=h + 500))


@pytest.mark.parametrize("s", [(1, 2), (31, 33), (0, 64), (0, 0), (1000, 17)])
def test_lengths_ragged_empty(s):
    run(shape(2, 32, s, seed=sum(s) + 501))


def test_scales_enter_latent_and_rotary_parts():
    # very different scales: a scale applied to the wrong part would fail
    run(shape(2, 32, (300, 45), seed=502), cs=0.004, rs=0.9)
    run(shape(2, 32, (300, 45), seed=503), cs=0.5, rs=0.01)


def test_other_dims_and_long_context():
    run(shape(19, 16, tuple(range(5, 5 + 19 * 7, 7)), seed=505, d_nope=64, d_v=32))
    run(shape(1, 128, (12000,), seed=506))


def test_schedule_mixed_paged():
    rng = np.random.default_rng(507)
    s = tuple(int(x) for x in rng.integers(0, 3000, size=40))
    run(shape(40, 32, s, paged=True, seed=507), sample=[0, 7, 13, 21, 39])


def test_paged_shuffled():
    run(shape(4, 32, (1, 16, 17, 700), paged=True, seed=508))


def test_deepseek_v3_full_size_sampled():
    sh = synth.configs()["deepseek_v3_mla"]
    run(sh, sample=[0, 17, sh.B - 1])


def test_peaked_logits_take_the_rescaling_path():
    # a late latent row along head 0's absorbed query (in code units): the
    # split holding it is recomputed by the merge kernel from the codes
    sh = shape(2, 128, (300, 5000), seed=509)
    cs, rs = 0.05, 0.05
    d = synth.draw_mla_fp8(sh, cs, rs, device=DEV)
    qt = torch.matmul(d["q_nope"][:, 0].float(), d["w_uk"][0].float())   # q~ of head 0
    for bi, t in ((0, 200), (1, 4000)):
        c = qt[bi] / qt[bi].norm() * 40.0
        r = d["q_rope"][bi, 0].float()
        kr = r / r.norm() * 40.0
        row = torch.cat([synth.fp8_codes(c, cs), synth.fp8_codes(kr, rs)])
        d["cache8"][bi, t] = row
    out, ul, lse = A.decode_mla(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["cache8"], d["s"],
                                c_scale=cs, r_scale=rs)
    torch.cuda.synchronize()
    check(d, sh, out, ul, lse, cs, rs)
    assert float(lse[0, 0]) > 50


def test_bad_arguments():
    sh = shape(1, 16, (10,), seed=510)
    d = synth.draw_mla_fp8(sh, CS, RS, device=DEV)
    out = torch.empty((1, 16, 128), dtype=torch.bfloat16, device=DEV)
    for cs, rs in ((0.0, 1.0), (1.0, -1.0), (float("inf"), 1.0)):
        rc = A.attn_decode_mla_absorbed_fp8(out, None, None, d["q_nope"], d["q_rope"], d["w_uk"],
                                            d["w_uv"], d["cache8"], cs, rs, d["s"], None, 0, 16, 0,
                                            1, sh.s_max, 16, 512, 64, 128, 128, 0.0, None, 0,
                                            check=False)
        assert rc == A.ATTN_EINVAL, (cs, rs, rc)


@pytest.mark.parametrize("paged", [False, True])
def test_append_bit_exact(paged):
    B, s_max, W = 5, 40, 576
    rng = np.random.default_rng(511)
    kv = torch.from_numpy(rng.standard_normal((B, W)).astype(np.float32) * 3).to(torch.bfloat16)
    kv[0, 0], kv[0, 1], kv[0, 513] = float("nan"), 1e6, -1e6   # NaN and saturation in both parts
    kv = kv.to(DEV)
    pos = np.array([0, 39, 16, 15, 7], np.int32)
    cs, rs = 0.02, 0.3
    if paged:
        nblk = B * 3
        perm = rng.permutation(nblk).astype(np.int32)
        bt = perm.reshape(B, 3)
        cache = torch.from_numpy(rng.integers(0, 256, size=(nblk, 16, W), dtype=np.uint8)).to(DEV)
        host = synth.host_bits(cache)
        A.kv_cache_append_mla_fp8(cache, kv, cs, rs, torch.from_numpy(pos).to(DEV),
                                  torch.from_numpy(bt).to(DEV), 3, 16, nblk, B, 48, 512, 64)
        want = oracle.kv_append_mla_fp8(host, synth.host_bits(kv.cpu()), cs, rs, pos, 512,
                                        block_table=bt)
    else:
        cache = torch.from_numpy(rng.integers(0, 256, size=(B, s_max, W), dtype=np.uint8)).to(DEV)
        host = synth.host_bits(cache)
        A.kv_cache_append_mla_fp8(cache, kv, cs, rs, torch.from_numpy(pos).to(DEV), None, 0, 16, 0,
                                  B, s_max, 512, 64)
        want = oracle.kv_append_mla_fp8(host, synth.host_bits(kv.cpu()), cs, rs, pos, 512)
    torch.cuda.synchronize()
    assert np.array_equal(synth.host_bits(cache), want)
