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


# ---- one scale pair per page (attn_decode_mla_absorbed_fp8_paged_scales) ----
def page_scales(n_blk, seed, lo=0.5 * CS, hi=1.5 * CS):
    """Per-page latent and rotary scales, unrelated across pages and parts
    (around the scale the codes were drawn with, so that the values stay
    O(1) like the other tests' and the bf16 bounds mean the same)."""
    rng = np.random.default_rng(seed)
    cs = rng.uniform(lo, hi, size=n_blk).astype(np.float32)
    rs = rng.uniform(lo, hi, size=n_blk).astype(np.float32)
    return cs, rs


def run_paged_scales(sh, sample=None, seed=0, poke=None):
    print(f"[mla-fp8-pages] B={sh.B} h={sh.h} s={list(sh.s)[:6]}", flush=True)
    d = synth.draw_mla_fp8(sh, CS, RS, device=DEV)
    n_blk = d["cache8"].shape[0]
    cs, rs = page_scales(n_blk, seed)
    if poke is not None:
        poke(d, cs, rs)
    out, ul, lse = A.decode_mla(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["cache8"], d["s"],
                                block_table=d["block_table"], s_max=sh.s_max,
                                c_scale=torch.from_numpy(cs).to(DEV),
                                r_scale=torch.from_numpy(rs).to(DEV))
    torch.cuda.synchronize()
    pool = synth.host_bits(d["cache8"])
    W = [synth.host_bits(d[k]) for k in ("w_uk", "w_uv")]
    for bi in (range(sh.B) if sample is None else sample):
        args = [synth.host_bits(d[k][bi:bi + 1]) for k in ("q_nope", "q_rope")]
        bt = d["block_table_host"][bi:bi + 1]
        ro, ru, rl = oracle.mla_absorbed_fp8_paged_scales(args[0], args[1], *W, pool, cs, rs,
                                                          np.array([int(sh.s[bi])], np.int32), bt)
        assert_close(to_f64(out[bi:bi + 1]), ro, 2, f"out b={bi}")
        assert_close(to_f64(ul[bi:bi + 1]), ru, 2, f"u_latent b={bi}")
        assert_lse_close(to_f64(lse[bi:bi + 1]), rl, 2, f"lse b={bi}")
    return d, out, ul, lse


@pytest.mark.parametrize("h", [16, 128])
def test_page_scales_heads(h):
    run_paged_scales(shape(3, h, (77, 300, 1025), paged=True, seed=h + 520), seed=h)


@pytest.mark.parametrize("s", [(0, 40), (1, 15), (16, 17), (33, 0)])
def test_page_scales_short_and_empty(s):
    run_paged_scales(shape(2, 32, s, paged=True, seed=sum(s) + 521), seed=sum(s))


def test_page_scales_mixed_lengths_long():
    rng = np.random.default_rng(522)
    s = tuple(int(x) for x in rng.integers(0, 6000, size=24)) + (20000,)
    run_paged_scales(shape(25, 64, s, paged=True, seed=522), sample=[0, 9, 24], seed=522)


def test_page_scales_peaked_logits_take_the_rescaling_path():
    sh = shape(2, 128, (300, 5000), paged=True, seed=523)

    def poke(d, cs, rs):
        # a spike of value length 40 in both parts (as the bf16 test), on a
        # page whose scales are set to 0.08: 500 code units
        qt = torch.matmul(d["q_nope"][:, 0].float(), d["w_uk"][0].float())
        tab = d["block_table_host"]
        for bi, t in ((0, 200), (1, 4000)):
            blk = int(tab[bi, t // 16])
            cs[blk] = rs[blk] = 0.08
            c = qt[bi] / qt[bi].norm() * 40.0
            r = d["q_rope"][bi, 0].float()
            kr = r / r.norm() * 40.0
            d["cache8"][blk, t % 16] = torch.cat([synth.fp8_codes(c, 0.08), synth.fp8_codes(kr, 0.08)])

    _, _, _, lse = run_paged_scales(sh, seed=523, poke=poke)
    assert float(lse[0, 0]) > 50            # the spike dominates head 0


def test_page_scales_paged_mla_full_size_sampled():
    sh = synth.configs()["paged_mla"]
    lens = np.asarray(sh.s)
    run_paged_scales(sh, sample=[int(np.argmin(lens)), int(np.argmax(lens))], seed=524)


def test_page_scales_append_bit_exact():
    B, W = 5, 576
    rng = np.random.default_rng(525)
    kv = torch.from_numpy(rng.standard_normal((B, W)).astype(np.float32) * 3).to(torch.bfloat16)
    kv[0, 0], kv[0, 1], kv[0, 513] = float("nan"), 1e6, -1e6
    kv = kv.to(DEV)
    pos = np.array([0, 39, 16, 15, 7], np.int32)
    nblk = B * 3
    bt = rng.permutation(nblk).astype(np.int32).reshape(B, 3)
    cs, rs = page_scales(nblk, 525, 0.005, 0.5)
    cache = torch.from_numpy(rng.integers(0, 256, size=(nblk, 16, W), dtype=np.uint8)).to(DEV)
    host = synth.host_bits(cache)
    A.kv_cache_append_mla_fp8_paged_scales(cache, kv, torch.from_numpy(cs).to(DEV),
                                           torch.from_numpy(rs).to(DEV),
                                           torch.from_numpy(pos).to(DEV),
                                           torch.from_numpy(bt).to(DEV), 3, 16, nblk, B, 48, 512, 64)
    want = oracle.kv_append_mla_fp8_paged_scales(host, synth.host_bits(kv.cpu()), cs, rs, pos, 512,
                                                 bt)
    torch.cuda.synchronize()
    assert np.array_equal(synth.host_bits(cache), want)


def test_page_scales_bad_arguments():
    sh = shape(1, 16, (10,), paged=True, seed=526)
    d = synth.draw_mla_fp8(sh, CS, RS, device=DEV)
    out = torch.empty((1, 16, 128), dtype=torch.bfloat16, device=DEV)
    sc = torch.ones(d["cache8"].shape[0], dtype=torch.float32, device=DEV)
    bt = d["block_table"]
    kw = dict(check=False)
    rc = A.attn_decode_mla_absorbed_fp8_paged_scales(out, None, None, d["q_nope"], d["q_rope"],
                                                     d["w_uk"], d["w_uv"], d["cache8"], None, sc,
                                                     d["s"], bt, bt.shape[1], 16,
                                                     d["cache8"].shape[0], 1, 16, 16, 512, 64, 128,
                                                     128, 0.0, None, 0, **kw)
    assert rc == A.ATTN_EINVAL
    rc = A.attn_decode_mla_absorbed_fp8_paged_scales(out, None, None, d["q_nope"], d["q_rope"],
                                                     d["w_uk"], d["w_uv"], d["cache8"], sc, sc,
                                                     d["s"], None, 0, 16, 0, 1, 16, 16, 512, 64,
                                                     128, 128, 0.0, None, 0, **kw)
    assert rc == A.ATTN_EINVAL
