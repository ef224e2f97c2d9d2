"""Pins for the oracle's merge of slice partials (oracle.merge_partials).

A sequence's tokens split into disjoint slices; each slice's decode gives its
own output o_k and log-sum-exp lse_k, and the merge must give the decode over
all tokens ("MLA: why one latent can replace a multi-head KV cache", section
on what FlashMLA solves: per-block maximum, normaliser and output combined
stably).  Checked against:
  * torch's library attention in float64 over the whole token range (the
    slices' partials come from torch too, so the oracle's decode is not
    involved);
  * closed forms: one slice is the identity; two slices with equal lse give
    the mean and lse + ln 2; empty slices (lse = -inf) change nothing; all
    slices empty give 0 and -inf;
  * the order of the slices does not matter.
A wrong sign in the weights, a missing normalisation, a dropped maximum or a
wrong lse fails at least one of these.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests._util import bf16_bits, widen


def torch_attn(q, K, V):
    """q [h,d], K/V [n,h,d] float64 -> (out [h,d], lse [h]); n = 0 gives 0, -inf."""
    h, d = q.shape
    if K.shape[0] == 0:
        return np.zeros((h, V.shape[2])), np.full(h, -np.inf)
    qt = torch.from_numpy(q)
    kt = torch.from_numpy(K).permute(1, 0, 2)          # [h,n,d]
    vt = torch.from_numpy(V).permute(1, 0, 2)
    z = torch.einsum("hd,hnd->hn", qt, kt) / math.sqrt(d)
    lse = torch.logsumexp(z, dim=1)
    out = torch.einsum("hn,hnd->hd", torch.softmax(z, dim=1), vt)
    return out.numpy(), lse.numpy()


def slice_partials(B, h, d, dv, s, cuts, seed):
    """Whole-range reference and per-slice partials for B sequences."""
    rng = np.random.default_rng(seed)
    n = len(cuts[0]) - 1
    o_parts = np.zeros((n, B, h, dv))
    lse_parts = np.zeros((n, B, h))
    whole_o = np.zeros((B, h, dv))
    whole_l = np.zeros((B, h))
    for bi in range(B):
        q = rng.standard_normal((h, d))
        K = rng.standard_normal((s[bi], h, d))
        V = rng.standard_normal((s[bi], h, dv))
        whole_o[bi], whole_l[bi] = torch_attn(q, K, V)
        for k in range(n):
            a, e = cuts[bi][k], cuts[bi][k + 1]
            o_parts[k, bi], lse_parts[k, bi] = torch_attn(q, K[a:e], V[a:e])
    return o_parts, lse_parts, whole_o, whole_l


@pytest.mark.parametrize("dv", [64, 128, 512])
def test_merge_of_slices_equals_whole_attention(dv):
    B, h, d = 3, 4, 64
    s = [300, 17, 1000]
    # slice boundaries, some slices empty
    cuts = [[0, 100, 100, 250, 300], [0, 0, 5, 17, 17], [0, 1, 999, 1000, 1000]]
    o_parts, lse_parts, whole_o, whole_l = slice_partials(B, h, d, dv, s, cuts, seed=1)
    out, lse = oracle.merge_partials(o_parts.astype(np.float32), lse_parts.astype(np.float32), 4)
    # the fp32 storage of the partials bounds the agreement
    assert np.max(np.abs(out - whole_o)) < 2e-6
    assert np.max(np.abs(lse - whole_l)) < 2e-5
    # bf16 partials: within bf16 rounding of each o_k
    out2, _ = oracle.merge_partials(bf16_bits(o_parts), lse_parts.astype(np.float32), 2)
    assert np.max(np.abs(out2 - whole_o)) < 1e-2


def test_single_slice_is_the_identity():
    rng = np.random.default_rng(2)
    o = rng.standard_normal((1, 2, 3, 128)).astype(np.float32)
    l = rng.standard_normal((1, 2, 3)).astype(np.float32) * 10
    out, lse = oracle.merge_partials(o, l, 4)
    assert np.array_equal(out, o[0].astype(np.float64))
    assert np.array_equal(lse, l[0].astype(np.float64))
    ob = bf16_bits(o)
    out, _ = oracle.merge_partials(ob, l, 2)
    assert np.array_equal(out, widen(ob[0]))


def test_equal_lse_gives_mean_and_ln2():
    rng = np.random.default_rng(3)
    o = rng.standard_normal((2, 1, 2, 64)).astype(np.float32)
    l = np.full((2, 1, 2), 3.25, dtype=np.float32)
    out, lse = oracle.merge_partials(o, l, 4)
    assert np.allclose(out, (o[0].astype(np.float64) + o[1]) / 2, rtol=0, atol=1e-15)
    assert np.allclose(lse, 3.25 + math.log(2.0), rtol=0, atol=1e-15)


def test_unequal_lse_closed_form():
    # weights e^2 : e^0 -> out = (e^2 o1 + o2) / (e^2 + 1)
    o = np.zeros((2, 1, 1, 2), dtype=np.float32)
    o[0, 0, 0] = [1.0, 0.0]
    o[1, 0, 0] = [0.0, 1.0]
    l = np.array([[[2.0]], [[0.0]]], dtype=np.float32)
    out, lse = oracle.merge_partials(o, l, 4)
    e2 = math.exp(2.0)
    assert np.allclose(out[0, 0], [e2 / (e2 + 1), 1 / (e2 + 1)], rtol=0, atol=1e-15)
    assert abs(lse[0, 0] - math.log(e2 + 1)) < 1e-15


def test_empty_slices_change_nothing():
    rng = np.random.default_rng(4)
    o = rng.standard_normal((3, 2, 4, 32)).astype(np.float32)
    l = rng.standard_normal((3, 2, 4)).astype(np.float32)
    ref, ref_l = oracle.merge_partials(o, l, 4)
    o2 = np.concatenate([o, rng.standard_normal((2, 2, 4, 32)).astype(np.float32)])
    l2 = np.concatenate([l, np.full((2, 2, 4), -np.inf, dtype=np.float32)])
    out, lse = oracle.merge_partials(o2, l2, 4)
    assert np.array_equal(out, ref) and np.array_equal(lse, ref_l)


def test_all_slices_empty():
    o = np.ones((3, 1, 2, 16), dtype=np.float32)
    l = np.full((3, 1, 2), -np.inf, dtype=np.float32)
    out, lse = oracle.merge_partials(o, l, 4)
    assert np.all(out == 0.0) and np.all(lse == -np.inf)


def test_slice_order_does_not_matter():
    rng = np.random.default_rng(5)
    o = rng.standard_normal((6, 2, 3, 64)).astype(np.float32)
    l = (rng.standard_normal((6, 2, 3)) * 5).astype(np.float32)
    perm = rng.permutation(6)
    a, la = oracle.merge_partials(o, l, 4)
    b, lb = oracle.merge_partials(o[perm], l[perm], 4)
    assert np.max(np.abs(a - b)) < 1e-14 and np.max(np.abs(la - lb)) < 1e-14


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.merge_partials(np.zeros((2, 1, 1, 4), np.float32), np.zeros((1, 1, 1), np.float32), 4)
