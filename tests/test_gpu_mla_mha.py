"""GPU parity of attn_decode_mla_mha -- MLA in MHA mode (explicit per-head
K/V, then plain multi-head attention over the causal prefix of each new
token) -- against the oracle's multi-token MLA decode, which computes the
same out and lse (pinned to torch's masked attention on the explicit
expansion).  Tolerances: the bf16 bounds of the other MLA tests (max-abs <=
2e-2, mean-abs <= 2e-3, rel-RMS <= 1e-2); the expanded K and V and the
probabilities are rounded to bf16 for the matrix cores, sums are fp32."""
import numpy as np
import pytest
import torch

import decode_attention_kv_attn_amd as A
import oracle
import synth
from tests._gpu import assert_close, assert_lse_close, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def shape(B, h, s, q_len, paged=False, seed=31):
    return synth.MlaShape("t", B=B, h=h, d_c=512, d_R=64, d_nope=128, d_v=128, s=tuple(s),
                          paged=paged, seed=seed, q_len=q_len)


def rows_of(d, sh, bi):
    n = int(sh.s[bi])
    if sh.paged:
        tab = d["block_table_host"][bi]
        nb = (n + sh.block_size - 1) // sh.block_size
        idx = torch.as_tensor(tab[:nb], dtype=torch.long, device=DEV)
        return d["cache"].index_select(0, idx).reshape(-1, sh.d_c + sh.d_R)[:max(n, 1)]
    return d["cache"][bi, :max(n, 1)]


def draw(sh):
    d = synth.draw_mla(sh, device=DEV)
    if sh.q_len == 1:   # the multi-token layout always has the q_len axis
        d["q_nope"], d["q_rope"] = d["q_nope"][:, None], d["q_rope"][:, None]
    return d


def run(sh, sample=None):
    print(f"[mla-mha] B={sh.B} q_len={sh.q_len} h={sh.h} s={list(sh.s)[:6]} paged={sh.paged}",
          flush=True)
    d = draw(sh)
    out, lse = A.decode_mla_mha(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["cache"],
                                d["s"], block_table=d.get("block_table"), s_max=sh.s_max)
    torch.cuda.synchronize()
    w = [synth.host_bits(d["w_uk"]), synth.host_bits(d["w_uv"])]
    for bi in (range(sh.B) if sample is None else sample):
        qn, qr = (synth.host_bits(d[k][bi:bi + 1]) for k in ("q_nope", "q_rope"))
        C = synth.host_bits(rows_of(d, sh, bi))[None]
        ro, _, rl = oracle.mla_absorbed_multi(qn, qr, *w, C, np.array([int(sh.s[bi])], np.int32))
        assert_close(to_f64(out[bi:bi + 1]), ro, 2, f"out b={bi}")
        assert_lse_close(to_f64(lse[bi:bi + 1]), rl, 2, f"lse b={bi}")
    return d, out, lse


@pytest.mark.parametrize("q_len", [1, 5, 64, 100, 300])
def test_query_block_lengths(q_len):
    run(shape(2, 16, (130, 777), q_len, seed=60 + q_len))


def test_all_heads_of_a_deepseek_layer():
    run(shape(2, 128, (300, 1500), 16, seed=61))


@pytest.mark.parametrize("s", [(0, 40), (3, 0), (1, 100)])
def test_sequences_shorter_than_the_query_block(s):
    _, out, lse = run(shape(2, 16, s, 8, seed=sum(s) + 62))
    for bi, n in enumerate(s):
        k = max(8 - n, 0)
        assert torch.all(out[bi, :k] == 0) and torch.all(torch.isneginf(lse[bi, :k]))


def test_paged_mixed():
    rng = np.random.default_rng(63)
    s = tuple(int(x) for x in rng.integers(0, 2500, size=12))
    run(shape(12, 32, s, 24, paged=True, seed=63), sample=[0, 4, 11])


def test_agrees_with_the_absorbed_kernel():
    # both forms of one layer on one input; each is within the bf16 bounds
    # of the oracle, and of each other
    sh = shape(3, 32, (64, 900, 2000), 12, seed=64)
    d = draw(sh)
    mo, ml = A.decode_mla_mha(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["cache"], d["s"])
    ao, _, al = A.decode_mla_multi(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["cache"],
                                   d["s"], want_latent=False)
    torch.cuda.synchronize()
    assert_close(to_f64(mo), to_f64(ao), 2, "MHA vs absorbed out")
    assert_lse_close(to_f64(ml), to_f64(al).astype(np.float64), 2, "MHA vs absorbed lse")


def test_long_context_sampled():
    run(shape(2, 128, (8192, 5000), 64, seed=65), sample=[1])
