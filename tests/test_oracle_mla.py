"""Pins for the MLA oracles (oracle.mla_absorbed, oracle.mla_explicit).

  * explicit expansion vs torch's library attention: k_i = [W_UK[i] c ; k_R],
    v_i = W_UV[i] c built with torch matmuls, then scaled_dot_product_attention
    in float64 with scale 1/sqrt(d_nope + d_R) ("Multi-Head Latent Attention
    (MLA): Mathematical Foundations", sections "Low-Rank Joint Key-Value
    Compression", "The Decoupled RoPE Solution" and "Value Output Matrix
    Absorption");
  * absorbed == explicit (both absorption identities: "Attention Logit Matrix
    Absorption" and "Value Output Matrix Absorption"; the same check is the
    "Absorption" step of the validation chain on the charlestar.github.io MLA
    page);
  * reduction to MQA: with d_nope = d_c and W_UK = W_UV = I the absorbed path
    is plain one-KV-head attention over the latent rows, so torch's library
    attention over [c | k_R] (values c) must give both out and u_latent, and
    so must the GQA oracle with one KV head ("MHA -> MQA -> GQA -> MLA",
    sections "Where h_kv comes from" and "Where the head count becomes
    bytes": an MLA layer decodes as one KV head shared by every query head);
  * paged == contiguous gathered, bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from tests._util import bf16_bits, gather_rows, mla_host, widen


def torch_explicit(d, scale=None):
    qn, qr = widen(d["q_nope"]), widen(d["q_rope"])
    C, wuk, wuv = widen(d["cache"]), widen(d["w_uk"]), widen(d["w_uv"])
    B, h, d_nope = qn.shape
    d_R = qr.shape[2]
    d_c = wuk.shape[2]
    d_v = wuv.shape[1]
    sc = 1.0 / np.sqrt(d_nope + d_R) if scale is None else scale
    out = np.zeros((B, h, d_v))
    lse = np.zeros((B, h))
    for bi in range(B):
        n = int(d["s"][bi])
        c = torch.from_numpy(C[bi, :n, :d_c])                        # [n, d_c]
        kr = torch.from_numpy(C[bi, :n, d_c:])                        # [n, d_R]
        kc = torch.matmul(torch.from_numpy(wuk), c.T.contiguous())    # [h, d_nope, n]
        v = torch.matmul(torch.from_numpy(wuv), c.T.contiguous())     # [h, d_v, n]
        k = torch.cat([kc.transpose(1, 2), kr.unsqueeze(0).expand(h, n, d_R)], dim=2)
        q = torch.cat([torch.from_numpy(qn[bi]), torch.from_numpy(qr[bi])], dim=1).unsqueeze(1)
        o = torch.nn.functional.scaled_dot_product_attention(
            q, k.contiguous(), v.transpose(1, 2).contiguous(), scale=sc)
        out[bi] = o[:, 0].numpy()
        z = torch.matmul(q, k.transpose(1, 2).contiguous())[:, 0] * sc
        lse[bi] = torch.logsumexp(z, dim=-1).numpy()
    return out, lse


SMALL = [
    # B, h, d_c, d_R, d_nope, d_v, s
    (2, 4, 32, 8, 16, 16, (5, 40)),
    (1, 8, 64, 16, 32, 24, (70,)),
    (3, 2, 16, 0, 8, 8, (1, 2, 33)),        # no RoPE segment
]


@pytest.mark.parametrize("B,h,d_c,d_R,d_nope,d_v,s", SMALL)
def test_explicit_matches_library_attention(B, h, d_c, d_R, d_nope, d_v, s):
    d = mla_host(B, h, d_c, d_R, d_nope, d_v, s, seed=41)
    out, lse = oracle.mla_explicit(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["cache"],
                                   d["s"])
    ref, ref_lse = torch_explicit(d)
    np.testing.assert_allclose(out, ref, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, atol=1e-12)


@pytest.mark.parametrize("B,h,d_c,d_R,d_nope,d_v,s", SMALL + [(2, 16, 128, 32, 64, 64, (64, 9))])
def test_absorbed_equals_explicit(B, h, d_c, d_R, d_nope, d_v, s):
    d = mla_host(B, h, d_c, d_R, d_nope, d_v, s, seed=43)
    args = (d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["cache"], d["s"])
    oa, ua, la = oracle.mla_absorbed(*args)
    oe, le = oracle.mla_explicit(*args)
    scale = np.max(np.abs(oe))
    assert np.max(np.abs(oa - oe)) <= 1e-10 * scale
    np.testing.assert_allclose(la, le, atol=1e-10)


def test_deepseek_v3_shape_reduced_absorbed_equals_explicit():
    # full head geometry (h=128, d_c=512, d_R=64, d_nope=d_v=128), short context
    d = mla_host(1, 128, 512, 64, 128, 128, (24,), seed=47)
    args = (d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["cache"], d["s"])
    oa, _, la = oracle.mla_absorbed(*args)
    oe, le = oracle.mla_explicit(*args)
    assert np.max(np.abs(oa - oe)) <= 1e-10 * np.max(np.abs(oe))
    np.testing.assert_allclose(la, le, atol=1e-10)


def test_default_scale_is_inverse_sqrt_of_nope_plus_rope():
    d = mla_host(1, 4, 32, 8, 16, 16, (20,), seed=53)
    args = (d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["cache"], d["s"])
    o1, _, _ = oracle.mla_absorbed(*args)
    o2, _, _ = oracle.mla_absorbed(*args, scale=1.0 / np.sqrt(16 + 8))
    assert np.array_equal(o1, o2)
    o3, _, _ = oracle.mla_absorbed(*args, scale=1.0 / np.sqrt(32 + 8))
    assert not np.allclose(o1, o3)


def test_identity_weights_reduce_to_mqa_over_latent():
    B, h, d_c, d_R = 2, 4, 32, 8
    d = mla_host(B, h, d_c, d_R, d_c, d_c, (11, 48), seed=59)
    eye = np.broadcast_to(np.eye(d_c, dtype=np.float32), (h, d_c, d_c))
    d["w_uk"] = bf16_bits(eye)
    d["w_uv"] = bf16_bits(eye)
    out, ul, lse = oracle.mla_absorbed(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"],
                                       d["cache"], d["s"])
    C = widen(d["cache"])
    q = np.concatenate([widen(d["q_nope"]), widen(d["q_rope"])], axis=2)
    sc = 1.0 / np.sqrt(d_c + d_R)
    for bi in range(B):
        n = int(d["s"][bi])
        k = torch.from_numpy(C[bi, :n]).unsqueeze(0).expand(h, n, d_c + d_R).contiguous()
        v = torch.from_numpy(C[bi, :n, :d_c]).unsqueeze(0).expand(h, n, d_c).contiguous()
        qt = torch.from_numpy(q[bi]).unsqueeze(1)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, k, v, scale=sc)[:, 0].numpy()
        np.testing.assert_allclose(out[bi], ref, atol=1e-12)
        np.testing.assert_allclose(ul[bi], ref, atol=1e-12)
        z = torch.matmul(qt, k.transpose(1, 2).contiguous())[:, 0] * sc
        np.testing.assert_allclose(lse[bi], torch.logsumexp(z, -1).numpy(), atol=1e-12)


def test_paged_shuffled_equals_contiguous_gather():
    s = (3, 16, 40)
    d = mla_host(3, 4, 32, 8, 16, 16, s, seed=61, paged=True)
    args = (d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"])
    op, up, lp = oracle.mla_absorbed(*args, d["cache"], d["s"], block_table=d["bt"])
    Cc = gather_rows(d["cache"], d["bt"], s, 16, 40)
    oc, uc, lc = oracle.mla_absorbed(*args, Cc, d["s"])
    assert np.array_equal(op, oc) and np.array_equal(up, uc) and np.array_equal(lp, lc)


def test_empty_sequence():
    d = mla_host(2, 4, 32, 8, 16, 16, (0, 7), seed=67)
    o, u, l = oracle.mla_absorbed(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["cache"],
                                  d["s"])
    assert np.all(o[0] == 0) and np.all(u[0] == 0) and np.all(np.isneginf(l[0]))
    assert np.all(np.isfinite(o[1]))


def test_identity_weights_reduce_to_the_gqa_oracle_with_one_kv_head():
    # With d_nope = d_c and W_UK = W_UV = I, absorbed MLA is MQA over the
    # latent rows ("MHA -> MQA -> GQA -> MLA", the MLA section: decode in the
    # absorbed form is MQA): keys [c | k_R], values c, queries [q_nope | q_rope],
    # one KV head.  The GQA oracle takes equal key and value widths, so the
    # values are padded with d_R zero columns, which come back as zeros.
    B, h, d_c, d_R = 2, 4, 32, 8
    d = mla_host(B, h, d_c, d_R, d_c, d_c, (9, 37), seed=71)
    eye = np.broadcast_to(np.eye(d_c, dtype=np.float32), (h, d_c, d_c))
    d["w_uk"] = bf16_bits(eye)
    d["w_uv"] = bf16_bits(eye)
    out, ul, lse = oracle.mla_absorbed(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"],
                                       d["cache"], d["s"])
    C = d["cache"]                                      # [B, s_max, d_c + d_R] bf16 bits
    K = np.ascontiguousarray(C[:, :, None, :])          # h_kv = 1
    V = np.zeros_like(K)
    V[:, :, 0, :d_c] = C[:, :, :d_c]
    q = np.ascontiguousarray(np.concatenate([d["q_nope"], d["q_rope"]], axis=2))
    go, gl = oracle.gqa_decode(q, K, V, d["s"], 2, scale=1.0 / np.sqrt(d_c + d_R))
    np.testing.assert_allclose(ul, go[:, :, :d_c], rtol=0, atol=1e-12)
    np.testing.assert_allclose(out, go[:, :, :d_c], rtol=0, atol=1e-12)
    assert np.all(go[:, :, d_c:] == 0.0)
    np.testing.assert_allclose(lse, gl, rtol=0, atol=1e-12)
