"""Pins for the multi-token MLA oracle (oracle.mla_absorbed_multi and its FP8 form).

q_len new tokens per sequence, all already in the cache: position j sits at
cache position s_b - q_len + j and sees the tokens up to and including itself
(the tokens a speculative step verifies; "MLA: why one latent can replace a
multi-head KV cache", charlestar.github.io, lists their count and the query
length among the inputs of MLA kernel selection, and its validation chain's
"Kernel" step compares outputs and log-sum-exp over those lengths).

  * torch's library attention on the explicit expansion (k_i = [W_UK[i] c ;
    k_R], v_i = W_UV[i] c, "Multi-Head Latent Attention (MLA): Mathematical
    Foundations", sections "Low-Rank Joint Key-Value Compression" and "The
    Decoupled RoPE Solution") with a causal mask whose diagonal sits at the
    last q_len cache positions;
  * every position equals a single-token decode over the truncated sequence
    (lengths computed here, in Python);
  * q_len = 1 is the single-token oracle, bit for bit;
  * a sequence shorter than q_len: its first q_len - s_b positions see
    nothing (zeros, lse = -inf);
  * paged == contiguous gathered, bit for bit;
  * FP8 cache with power-of-two scales == the bf16 oracle on the decoded
    values (every E4M3 value times a power of two is a bf16 value).
"""
import numpy as np
import pytest
import torch

import oracle
from tests._util import gather_rows, mla_host, widen


def torch_masked_explicit(d, q_len):
    """Explicit K/V expansion + torch SDPA with the causal mask, float64."""
    qn, qr = widen(d["q_nope"]), widen(d["q_rope"])       # [B, q_len, h, .]
    C, wuk, wuv = widen(d["cache"]), widen(d["w_uk"]), widen(d["w_uv"])
    B, _, h, d_nope = qn.shape
    d_R = qr.shape[3]
    d_c = wuk.shape[2]
    d_v = wuv.shape[1]
    sc = 1.0 / np.sqrt(d_nope + d_R)
    out = np.zeros((B, q_len, h, d_v))
    lse = np.full((B, q_len, h), -np.inf)
    for bi in range(B):
        n = int(d["s"][bi])
        if n == 0:
            continue
        c = torch.from_numpy(C[bi, :n, :d_c])
        kr = torch.from_numpy(C[bi, :n, d_c:])
        kc = torch.matmul(torch.from_numpy(wuk), c.T.contiguous())    # [h, d_nope, n]
        v = torch.matmul(torch.from_numpy(wuv), c.T.contiguous())     # [h, d_v, n]
        k = torch.cat([kc.transpose(1, 2), kr.unsqueeze(0).expand(h, n, d_R)], dim=2)
        q = torch.cat([torch.from_numpy(qn[bi]), torch.from_numpy(qr[bi])], dim=2)
        q = q.transpose(0, 1).contiguous()                           # [h, q_len, d]
        pos = torch.arange(q_len).unsqueeze(1) + (n - q_len)         # cache position of query j
        mask = torch.arange(n).unsqueeze(0) <= pos                   # [q_len, n]
        seen = mask.any(dim=1)
        z = torch.matmul(q, k.transpose(1, 2).contiguous()) * sc     # [h, q_len, n]
        z = z.masked_fill(~mask, float("-inf"))
        o = torch.nn.functional.scaled_dot_product_attention(
            q[:, seen], k.contiguous(), v.transpose(1, 2).contiguous(), attn_mask=mask[seen],
            scale=sc)
        out[bi][seen.numpy()] = o.transpose(0, 1).numpy()
        lse[bi][seen.numpy()] = torch.logsumexp(z[:, seen], dim=-1).transpose(0, 1).numpy()
    return out, lse


CASES = [
    # B, h, d_c, d_R, d_nope, d_v, s, q_len
    (2, 4, 32, 8, 16, 16, (9, 40), 2),
    (1, 8, 64, 16, 32, 24, (70,), 4),
    (3, 2, 16, 0, 8, 8, (8, 12, 33), 8),           # no RoPE segment
    (2, 4, 32, 8, 16, 16, (3, 21), 5),             # first sequence shorter than q_len
]


def _args(d):
    return d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["cache"], d["s"]


@pytest.mark.parametrize("B,h,d_c,d_R,d_nope,d_v,s,q_len", CASES)
def test_matches_masked_library_attention(B, h, d_c, d_R, d_nope, d_v, s, q_len):
    d = mla_host(B, h, d_c, d_R, d_nope, d_v, s, seed=101, q_len=q_len)
    out, _, lse = oracle.mla_absorbed_multi(*_args(d))
    ref, ref_lse = torch_masked_explicit(d, q_len)
    assert np.max(np.abs(out - ref)) <= 1e-10 * max(np.max(np.abs(ref)), 1.0)
    np.testing.assert_allclose(lse, ref_lse, atol=1e-10)


@pytest.mark.parametrize("B,h,d_c,d_R,d_nope,d_v,s,q_len", CASES)
def test_each_position_is_a_single_token_decode_of_the_truncated_sequence(
        B, h, d_c, d_R, d_nope, d_v, s, q_len):
    d = mla_host(B, h, d_c, d_R, d_nope, d_v, s, seed=103, q_len=q_len)
    out, ul, lse = oracle.mla_absorbed_multi(*_args(d))
    for j in range(q_len):
        s_j = np.maximum(np.asarray(s) - (q_len - 1 - j), 0).astype(np.int32)
        qn = np.ascontiguousarray(d["q_nope"][:, j])
        qr = np.ascontiguousarray(d["q_rope"][:, j])
        o1, u1, l1 = oracle.mla_absorbed(qn, qr, d["w_uk"], d["w_uv"], d["cache"], s_j)
        assert np.array_equal(out[:, j], o1) and np.array_equal(ul[:, j], u1)
        assert np.array_equal(lse[:, j], l1)


def test_q_len_one_is_the_single_token_oracle():
    d = mla_host(3, 4, 32, 8, 16, 16, (0, 5, 40), seed=107)
    o1, u1, l1 = oracle.mla_absorbed(*_args(d))
    om, um, lm = oracle.mla_absorbed_multi(d["q_nope"][:, None], d["q_rope"][:, None],
                                           *_args(d)[2:])
    assert np.array_equal(om[:, 0], o1) and np.array_equal(um[:, 0], u1)
    assert np.array_equal(lm[:, 0], l1)


def test_positions_before_a_short_sequence_see_nothing():
    q_len = 6
    d = mla_host(3, 4, 32, 8, 16, 16, (0, 2, 6), seed=109, q_len=q_len)
    out, ul, lse = oracle.mla_absorbed_multi(*_args(d))
    assert np.all(out[0] == 0) and np.all(ul[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(out[1, :4] == 0) and np.all(np.isneginf(lse[1, :4]))
    assert np.all(np.isfinite(lse[1, 4:])) and np.all(np.isfinite(lse[2]))
    # position 0 of the sequence of length 2 sees exactly one token: softmax of
    # one score is 1, so u~ is that token's latent row and lse its score
    c0 = widen(d["cache"])[1, 0]
    np.testing.assert_array_equal(ul[1, 4], np.broadcast_to(c0[:32], (4, 32)))


def test_paged_shuffled_equals_contiguous_gather():
    s, q_len = (3, 16, 40), 4
    d = mla_host(3, 4, 32, 8, 16, 16, s, seed=113, paged=True, q_len=q_len)
    a = (d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"])
    op, up, lp = oracle.mla_absorbed_multi(*a, d["cache"], d["s"], block_table=d["bt"])
    oc, uc, lc = oracle.mla_absorbed_multi(*a, gather_rows(d["cache"], d["bt"], s, 16, 40),
                                           d["s"])
    assert np.array_equal(op, oc) and np.array_equal(up, uc) and np.array_equal(lp, lc)


def test_fp8_power_of_two_scales_equal_bf16_on_decoded_values():
    from synth import MlaShape, draw_mla_fp8, host_bits
    q_len, c_s, r_s = 3, 0.25, 2.0
    sh = MlaShape("t", B=2, h=4, d_c=32, d_R=8, d_nope=16, d_v=16, s=(5, 30), seed=117,
                  q_len=q_len)
    d = draw_mla_fp8(sh, c_s, r_s)
    codes = d["cache8"].numpy()
    dec = oracle.fp8_decode(codes)
    vals = np.concatenate([dec[..., :32] * c_s, dec[..., 32:] * r_s], axis=-1)
    bits = host_bits(torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16))
    assert np.array_equal(widen(bits), vals)          # exact in bf16
    q = [host_bits(d[k]) for k in ("q_nope", "q_rope", "w_uk", "w_uv")]
    o8, u8, l8 = oracle.mla_absorbed_multi_fp8(*q, codes, c_s, r_s, d["s_host"])
    ob, ub, lb = oracle.mla_absorbed_multi(*q, bits, d["s_host"])
    assert np.array_equal(o8, ob) and np.array_equal(u8, ub) and np.array_equal(l8, lb)
