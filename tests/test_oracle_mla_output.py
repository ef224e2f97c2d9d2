"""Pins for the MLA output-projection oracle (oracle.mla_output).

"Multi-Head Latent Attention (MLA): Mathematical Foundations" (llms.blog),
section "Value Output Matrix Absorption": the heads are aggregated by
W_O = [W_O^1 .. W_O^h] in R^{d x h d_v}, o_t = sum_i W_O^i u_{t,i}, and the
same sum regrouped as sum_i (W_O^i W_UV,i) u~_{t,i} with the merged weight.

  * torch's library attention on the explicit K/V expansion, heads
    concatenated and multiplied by W_O^T (torch matmul, float64);
  * the regrouped (merged-weight) form from the absorbed latent sums;
  * W_O = I (d_model = h d_v) returns the concatenated head outputs exactly;
  * several new tokens per sequence: each position is the projection of the
    multi-token decode's heads;
  * lse is the decode's.
"""
import numpy as np
import pytest
import torch

import oracle
from tests._util import bf16_bits, mla_host, widen
from tests.test_oracle_mla import torch_explicit


def with_w_o(d, d_model, seed):
    h, d_v = d["w_uv"].shape[0], d["w_uv"].shape[1]
    rng = np.random.default_rng(seed)
    d["w_o"] = bf16_bits(rng.standard_normal((d_model, h * d_v)).astype(np.float32)
                         / np.sqrt(h * d_v))
    return d


SMALL = [
    # B, h, d_c, d_R, d_nope, d_v, s, d_model
    (2, 4, 32, 8, 16, 16, (5, 40), 48),
    (1, 8, 64, 16, 32, 24, (70,), 40),
    (3, 2, 16, 0, 8, 8, (1, 2, 33), 24),
]


def _args(d):
    return d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["w_o"], d["cache"], d["s"]


@pytest.mark.parametrize("B,h,d_c,d_R,d_nope,d_v,s,d_model", SMALL)
def test_matches_library_attention_then_projection(B, h, d_c, d_R, d_nope, d_v, s, d_model):
    d = with_w_o(mla_host(B, h, d_c, d_R, d_nope, d_v, s, seed=131), d_model, 1)
    o, lse = oracle.mla_output(*_args(d))
    heads, ref_lse = torch_explicit(d)                               # [B, h, d_v]
    ref = torch.matmul(torch.from_numpy(heads.reshape(B, h * d_v)),
                       torch.from_numpy(widen(d["w_o"])).T.contiguous()).numpy()
    assert np.max(np.abs(o - ref)) <= 1e-10 * np.max(np.abs(ref))
    np.testing.assert_allclose(lse, ref_lse, atol=1e-10)


@pytest.mark.parametrize("B,h,d_c,d_R,d_nope,d_v,s,d_model", SMALL)
def test_merged_weight_grouping_agrees(B, h, d_c, d_R, d_nope, d_v, s, d_model):
    d = with_w_o(mla_host(B, h, d_c, d_R, d_nope, d_v, s, seed=137), d_model, 2)
    o, _ = oracle.mla_output(*_args(d))
    _, ut, _ = oracle.mla_absorbed(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["cache"],
                                   d["s"])
    wo = widen(d["w_o"]).reshape(d_model, h, d_v)
    wuv = widen(d["w_uv"])                                            # [h, d_v, d_c]
    w_abs = np.stack([wo[:, i] @ wuv[i] for i in range(h)], axis=1)   # [d_model, h, d_c]
    merged = np.einsum("nic,bic->bn", w_abs, ut)
    assert np.max(np.abs(o - merged)) <= 1e-10 * np.max(np.abs(merged))


def test_identity_projection_returns_concatenated_heads():
    B, h, d_v = 2, 4, 16
    d = mla_host(B, h, 32, 8, 16, d_v, (9, 33), seed=139)
    d["w_o"] = bf16_bits(np.eye(h * d_v, dtype=np.float32))
    o, lse = oracle.mla_output(*_args(d))
    heads, _, l1 = oracle.mla_absorbed(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"],
                                       d["cache"], d["s"])
    assert np.array_equal(o, heads.reshape(B, h * d_v))
    assert np.array_equal(lse, l1)


def test_multi_token_positions_project_their_heads():
    q_len, d_model = 3, 40
    d = with_w_o(mla_host(2, 4, 32, 8, 16, 16, (2, 30), seed=149, q_len=q_len), d_model, 3)
    o, lse = oracle.mla_output(*_args(d))
    heads, _, lm = oracle.mla_absorbed_multi(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"],
                                             d["cache"], d["s"])
    ref = heads.reshape(2, q_len, -1) @ widen(d["w_o"]).T
    assert o.shape == (2, q_len, d_model)
    assert np.max(np.abs(o - ref)) <= 1e-12 * np.max(np.abs(ref))
    assert np.array_equal(lse, lm)
    assert np.all(o[0, 0] == 0)      # position 0 of a 2-token sequence with 3 new tokens
