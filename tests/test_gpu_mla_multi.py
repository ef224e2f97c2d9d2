"""GPU parity of attn_decode_mla_absorbed_multi(_fp8) -- q_len new tokens per
sequence, causal among themselves -- against the oracle's multi-token MLA
decode (pinned to torch's masked attention on the explicit K/V expansion).
Tolerances as the single-token MLA tests (bf16: max-abs <= 2e-2, mean-abs <=
2e-3, rel-RMS <= 1e-2): every (sequence, position) pair is one query row of
the same kernels."""
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


def shape(B, h, s, q_len, paged=False, seed=31, d_nope=128, d_v=128):
    return synth.MlaShape("t", B=B, h=h, d_c=512, d_R=64, d_nope=d_nope, d_v=d_v, s=tuple(s),
                          paged=paged, seed=seed, q_len=q_len)


def rows_of(cache, sh, d, bi):
    n = int(sh.s[bi])
    if sh.paged:
        tab = d["block_table_host"][bi]
        nb = (n + sh.block_size - 1) // sh.block_size
        idx = torch.as_tensor(tab[:nb], dtype=torch.long, device=DEV)
        return cache.index_select(0, idx).reshape(-1, sh.d_c + sh.d_R)[:max(n, 1)]
    return cache[bi, :max(n, 1)]


def run(sh, sample=None, fp8=False):
    print(f"[mla-multi] B={sh.B} q_len={sh.q_len} h={sh.h} s={list(sh.s)[:6]} paged={sh.paged} "
          f"fp8={fp8}", flush=True)
    if fp8:
        d = synth.draw_mla_fp8(sh, CS, RS, device=DEV)
        cache, kw = d["cache8"], dict(c_scale=CS, r_scale=RS)
    else:
        d = synth.draw_mla(sh, device=DEV)
        cache, kw = d["cache"], {}
    out, ul, lse = A.decode_mla_multi(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], cache,
                                      d["s"], block_table=d.get("block_table"), s_max=sh.s_max,
                                      **kw)
    torch.cuda.synchronize()
    w = [synth.host_bits(d["w_uk"]), synth.host_bits(d["w_uv"])]
    for bi in (range(sh.B) if sample is None else sample):
        n = int(sh.s[bi])
        qn, qr = (synth.host_bits(d[k][bi:bi + 1]) for k in ("q_nope", "q_rope"))
        C = synth.host_bits(rows_of(cache, sh, d, bi))[None]
        if fp8:
            ro, ru, rl = oracle.mla_absorbed_multi_fp8(qn, qr, *w, C, CS, RS,
                                                       np.array([n], np.int32))
        else:
            ro, ru, rl = oracle.mla_absorbed_multi(qn, qr, *w, C, np.array([n], np.int32))
        assert_close(to_f64(out[bi:bi + 1]), ro, 2, f"out b={bi}")
        assert_close(to_f64(ul[bi:bi + 1]), ru, 2, f"u_latent b={bi}")
        assert_lse_close(to_f64(lse[bi:bi + 1]), rl, 2, f"lse b={bi}")
    return d, out, ul, lse


@pytest.mark.parametrize("q_len", [2, 3, 4, 8])
def test_query_lengths(q_len):
    run(shape(3, 32, (77, 300, 1025), q_len, seed=10 + q_len))


@pytest.mark.parametrize("s", [(0, 5), (1, 2), (3, 0), (4, 33)])
def test_sequences_shorter_than_q_len(s):
    # positions before a sequence's first token see nothing: 0 and -inf
    _, out, ul, lse = run(shape(2, 16, s, 4, seed=sum(s) + 3))
    for bi, n in enumerate(s):
        k = max(4 - n, 0)
        assert torch.all(out[bi, :k] == 0) and torch.all(ul[bi, :k] == 0)
        assert torch.all(torch.isneginf(lse[bi, :k]))


def test_long_context_split_over_workgroups():
    run(shape(1, 128, (12000,), 2, seed=21))


def test_paged_mixed():
    rng = np.random.default_rng(22)
    s = tuple(int(x) for x in rng.integers(0, 3000, size=20))
    run(shape(20, 32, s, 3, paged=True, seed=22), sample=[0, 5, 11, 19])


@pytest.mark.parametrize("paged", [False, True])
def test_fp8_cache(paged):
    run(shape(3, 64, (9, 700, 2048), 4, paged=paged, seed=23 + paged), fp8=True)


def test_q_len_one_equals_single_token_entry_point():
    sh = shape(5, 64, (0, 1, 40, 777, 3000), 1, seed=24)
    d = synth.draw_mla(sh, device=DEV)
    a = A.decode_mla(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["cache"], d["s"])
    b = A.decode_mla_multi(d["q_nope"][:, None], d["q_rope"][:, None], d["w_uk"], d["w_uv"],
                           d["cache"], d["s"])
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0][:, 0].view(torch.int16))
    assert torch.equal(a[1], b[1][:, 0]) and torch.equal(a[2], b[2][:, 0])


def test_q_len_bounds_rejected():
    sh = shape(1, 16, (40,), 2, seed=25)
    d = synth.draw_mla(sh, device=DEV)
    B, h = 1, 16
    out = torch.empty((B, 2, h, 128), dtype=torch.bfloat16, device=DEV)
    for q_len in (0, 1025):
        rc = A.attn_decode_mla_absorbed_multi(out, None, None, out, out, d["w_uk"], d["w_uv"],
                                              d["cache"], d["s"], None, 0, 16, 0, B, q_len, 40,
                                              h, 512, 64, 128, 128, 2, 0.0, None, 0, check=False)
        assert rc == A.ATTN_EINVAL
    assert A.attn_decode_mla_multi_workspace_bytes(B, 1025, h, 512, 64) == 0


def test_deepseek_v3_full_size_two_tokens_sampled():
    base = synth.configs()["deepseek_v3_mla"]
    sh = shape(base.B, base.h, base.s, 2, seed=base.seed)
    run(sh, sample=[0, sh.B - 1])


def test_long_query_block_paged():
    # 96 positions per sequence: 192 query rows, several of them seeing nothing
    run(shape(2, 16, (50, 900), 96, paged=True, seed=26), sample=[0, 1])
