"""Pins for the GQA / MQA / MHA oracle (oracle.gqa_decode).

Each check is independent of the oracle's own code:
  * torch's library attention (scaled_dot_product_attention, float64, CPU)
    after repeating each KV head over its g query heads -- the broadcast of
    "MHA -> MQA -> GQA -> MLA", opening section;
  * closed forms: one token gives that token's value row; identical keys give
    the mean of V; V -> a V + c gives a o + c;
  * invariants: token permutation; splitting the token range and merging
    the two partial results through their lse equals the whole (the online
    softmax merge named in "MLA: why one latent can replace a multi-head KV
    cache", section on what FlashMLA solves);
  * the head map: query head i reads KV head floor(i / g);
  * paged through a shuffled block table == the contiguous gathered image,
    bit for bit ("What a paged KV cache block holds").
A dropped scale, a wrong head index, a transposed operand, a missing max
subtraction or a wrong lse all fail at least one of these.
"""
import numpy as np
import pytest
import torch

import oracle
from tests._util import gather_rows, gqa_host, stored, widen


def torch_gqa(q, K, V, s, scale=None):
    """Library attention in float64 per sequence; returns (out, lse)."""
    q, K, V = widen(q), widen(K), widen(V)
    B, h, d = q.shape
    h_kv = K.shape[2]
    g = h // h_kv
    out = np.zeros((B, h, d))
    lse = np.zeros((B, h))
    for bi in range(B):
        n = int(s[bi])
        qt = torch.from_numpy(q[bi]).unsqueeze(1)                          # [h,1,d]
        kt = torch.from_numpy(K[bi, :n]).permute(1, 0, 2).repeat_interleave(g, 0)  # [h,n,d]
        vt = torch.from_numpy(V[bi, :n]).permute(1, 0, 2).repeat_interleave(g, 0)
        sc = (1.0 / np.sqrt(d)) if scale is None else scale
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=sc)
        out[bi] = o[:, 0].numpy()
        z = torch.matmul(qt, kt.transpose(1, 2).contiguous()) * sc          # [h,1,n]
        lse[bi] = torch.logsumexp(z[:, 0], dim=-1).numpy()
    return out, lse


CASES = [
    # B, h, h_kv, d_h, s, b
    (2, 8, 2, 64, (100, 256), 4),      # the tiny fp32 workload shape
    (3, 4, 4, 32, (1, 17, 40), 4),     # MHA (g = 1), a one-token sequence
    (2, 8, 1, 16, (33, 64), 2),        # MQA, bf16 storage
    (2, 16, 2, 64, (70, 5), 2),        # GQA g = 8, bf16
]


@pytest.mark.parametrize("B,h,h_kv,d_h,s,b", CASES)
def test_matches_library_attention(B, h, h_kv, d_h, s, b):
    d = gqa_host(B, h, h_kv, d_h, s, b, seed=11)
    out, lse = oracle.gqa_decode(d["q"], d["K"], d["V"], d["s"], b)
    ref, ref_lse = torch_gqa(d["q"], d["K"], d["V"], d["s"])
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_explicit_scale_is_used():
    d = gqa_host(2, 4, 2, 32, (9, 20), 4, seed=3)
    out, lse = oracle.gqa_decode(d["q"], d["K"], d["V"], d["s"], 4, scale=0.37)
    ref, ref_lse = torch_gqa(d["q"], d["K"], d["V"], d["s"], scale=0.37)
    np.testing.assert_allclose(out, ref, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, atol=1e-12)


def test_single_token_returns_its_value_row():
    d = gqa_host(2, 8, 2, 64, (1, 1), 4, seed=5)
    out, lse = oracle.gqa_decode(d["q"], d["K"], d["V"], d["s"], 4)
    q, K, V = widen(d["q"]), widen(d["K"]), widen(d["V"])
    for bi in range(2):
        for i in range(8):
            j = i // 4
            assert np.array_equal(out[bi, i], V[bi, 0, j])
            z0 = np.dot(q[bi, i], K[bi, 0, j]) / 8.0
            assert abs(lse[bi, i] - z0) < 1e-12


def test_identical_keys_give_mean_of_values():
    d = gqa_host(2, 4, 2, 32, (50, 128), 4, seed=7)
    K = d["K"].copy()
    K[:] = K[:, :1]                       # every token has token 0's key
    out, lse = oracle.gqa_decode(d["q"], K, d["V"], d["s"], 4)
    V = widen(d["V"])
    q = widen(d["q"])
    for bi, n in enumerate(d["s"]):
        for i in range(4):
            j = i // 2
            np.testing.assert_allclose(out[bi, i], V[bi, :n, j].mean(axis=0), atol=1e-12)
            z = np.dot(q[bi, i], widen(K)[bi, 0, j]) / np.sqrt(32)
            assert abs(lse[bi, i] - (z + np.log(n))) < 1e-12


def test_value_affine_map():
    d = gqa_host(2, 8, 4, 32, (31, 64), 4, seed=9)
    # values with 8 significant bits, so 2 V + c (c in steps of 1/16) is exact in fp32
    V = widen(stored(d["V"], 2)).astype(np.float32)
    out, _ = oracle.gqa_decode(d["q"], d["K"], V, d["s"], 4)
    c = (np.arange(32, dtype=np.float32) - 16) / np.float32(16)
    V2 = (V * np.float32(2.0) + c).astype(np.float32)
    assert np.array_equal(V2.astype(np.float64), 2.0 * V.astype(np.float64) + c)
    out2, _ = oracle.gqa_decode(d["q"], d["K"], V2, d["s"], 4)
    np.testing.assert_allclose(out2, 2.0 * out + c, atol=1e-12)


def test_token_permutation_invariance():
    d = gqa_host(1, 8, 2, 64, (200,), 2, seed=13)
    out, lse = oracle.gqa_decode(d["q"], d["K"], d["V"], d["s"], 2)
    perm = np.random.default_rng(0).permutation(200)
    out2, lse2 = oracle.gqa_decode(d["q"], d["K"][:, perm], d["V"][:, perm], d["s"], 2)
    np.testing.assert_allclose(out2, out, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, atol=1e-13)


@pytest.mark.parametrize("cut", [1, 37, 128, 199])
def test_split_and_lse_merge_equals_whole(cut):
    d = gqa_host(1, 8, 2, 64, (200,), 2, seed=17)
    q, K, V = d["q"], d["K"], d["V"]
    out, lse = oracle.gqa_decode(q, K, V, d["s"], 2)
    o1, l1 = oracle.gqa_decode(q, np.ascontiguousarray(K[:, :cut]),
                               np.ascontiguousarray(V[:, :cut]), [cut], 2)
    o2, l2 = oracle.gqa_decode(q, np.ascontiguousarray(K[:, cut:]),
                               np.ascontiguousarray(V[:, cut:]), [200 - cut], 2)
    m = np.maximum(l1, l2)
    w1, w2 = np.exp(l1 - m), np.exp(l2 - m)
    merged = (w1[..., None] * o1 + w2[..., None] * o2) / (w1 + w2)[..., None]
    np.testing.assert_allclose(merged, out, atol=1e-12)
    np.testing.assert_allclose(m + np.log(w1 + w2), lse, atol=1e-12)


def test_query_head_i_reads_kv_head_i_div_g():
    B, h, h_kv, d_h = 1, 12, 3, 16
    d = gqa_host(B, h, h_kv, d_h, (40,), 4, seed=19)
    V = np.zeros_like(d["V"])
    for j in range(h_kv):
        V[:, :, j, :] = float(j + 1)
    out, _ = oracle.gqa_decode(d["q"], d["K"], V, d["s"], 4)
    for i in range(h):
        assert np.all(np.abs(out[0, i] - (i // (h // h_kv) + 1)) < 1e-12)


def test_g1_equals_mha_via_library():
    d = gqa_host(2, 6, 6, 32, (10, 64), 2, seed=23)
    out, _ = oracle.gqa_decode(d["q"], d["K"], d["V"], d["s"], 2)
    ref, _ = torch_gqa(d["q"], d["K"], d["V"], d["s"])
    np.testing.assert_allclose(out, ref, atol=1e-12)


@pytest.mark.parametrize("b", [2, 4])
def test_paged_shuffled_equals_contiguous_gather(b):
    s = (1, 16, 17, 100)
    d = gqa_host(4, 8, 2, 32, s, b, seed=29, paged=True)
    out_p, lse_p = oracle.gqa_decode(d["q"], d["K"], d["V"], d["s"], b, block_table=d["bt"])
    Kc = gather_rows(d["K"], d["bt"], s, 16, 100)
    Vc = gather_rows(d["V"], d["bt"], s, 16, 100)
    out_c, lse_c = oracle.gqa_decode(d["q"], Kc, Vc, d["s"], b)
    assert np.array_equal(out_p, out_c)
    assert np.array_equal(lse_p, lse_c)


def test_empty_sequence_gives_zero_and_minus_inf():
    d = gqa_host(2, 4, 2, 16, (0, 5), 4, seed=31)
    out, lse = oracle.gqa_decode(d["q"], d["K"], d["V"], d["s"], 4)
    assert np.all(out[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(out[1]))


def test_rejects_indivisible_heads_and_bad_lengths():
    d = gqa_host(1, 6, 3, 16, (4,), 4, seed=1)
    q = d["q"][:, :5].copy()                   # h = 5, h_kv = 3
    with pytest.raises(ValueError):
        oracle.gqa_decode(q, d["K"], d["V"], d["s"], 4)
    with pytest.raises(ValueError):
        oracle.gqa_decode(d["q"], d["K"], d["V"], [5], 4)    # s > s_max


def test_zero_query_gives_mean_of_values():
    # q = 0 makes every score 0: the softmax is uniform over the s_b tokens,
    # so each head returns the plain mean of its KV head's value rows and
    # lse = ln s_b
    d = gqa_host(2, 8, 2, 32, (13, 96), 4, seed=37)
    q = np.zeros_like(d["q"])
    out, lse = oracle.gqa_decode(q, d["K"], d["V"], d["s"], 4)
    V = widen(d["V"])
    for bi, n in enumerate(d["s"]):
        for i in range(8):
            np.testing.assert_allclose(out[bi, i], V[bi, :n, i // 4].mean(axis=0), atol=1e-12)
            assert abs(lse[bi, i] - np.log(n)) < 1e-12


def _mha_loop(q, K, V, s, scale):
    """An independently written MHA decode: plain Python loops per head, a
    max-subtracted softmax over the token list, float64 throughout."""
    B, h, d = q.shape
    out = np.zeros((B, h, d))
    lse = np.zeros((B, h))
    for bi in range(B):
        for i in range(h):
            z = [scale * float(np.dot(q[bi, i], K[bi, t, i])) for t in range(int(s[bi]))]
            m = max(z)
            w = [np.exp(x - m) for x in z]
            tot = sum(w)
            acc = np.zeros(d)
            for t, wt in enumerate(w):
                acc += wt * V[bi, t, i]
            out[bi, i] = acc / tot
            lse[bi, i] = m + np.log(tot)
    return out, lse


def test_g1_equals_independent_mha_loop():
    # GQA with g = 1 is MHA ("MHA -> MQA -> GQA -> MLA", opening section)
    d = gqa_host(2, 5, 5, 16, (7, 31), 4, seed=41)
    out, lse = oracle.gqa_decode(d["q"], d["K"], d["V"], d["s"], 4)
    ref, ref_lse = _mha_loop(widen(d["q"]), widen(d["K"]), widen(d["V"]), d["s"], 1.0 / 4.0)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-13)


def test_shift_of_all_scores_moves_only_lse():
    # Adding one vector u to every key of an MHA head adds scale * q . u to
    # every score of that head: the softmax, hence o, is unchanged and lse
    # moves by exactly that constant.  Values are small integers over 8 so
    # K + u is exact in fp32.
    rng = np.random.default_rng(43)
    B, h, d_h, s = 1, 3, 16, (40,)
    q = (rng.integers(-8, 9, (B, h, d_h)) / 8).astype(np.float32)
    K = (rng.integers(-8, 9, (B, s[0], h, d_h)) / 8).astype(np.float32)
    V = rng.standard_normal((B, s[0], h, d_h)).astype(np.float32)
    u = (rng.integers(-8, 9, (h, d_h)) / 8).astype(np.float32)
    K2 = (K + u[None, None]).astype(np.float32)
    assert np.array_equal(K2.astype(np.float64), K.astype(np.float64) + u.astype(np.float64))
    o1, l1 = oracle.gqa_decode(q, K, V, s, 4)
    o2, l2 = oracle.gqa_decode(q, K2, V, s, 4)
    shift = np.einsum("bhd,hd->bh", q.astype(np.float64), u.astype(np.float64)) / 4.0
    np.testing.assert_allclose(o2, o1, atol=1e-13)
    np.testing.assert_allclose(l2, l1 + shift, atol=1e-12)
    assert np.max(np.abs(shift)) > 0.1   # the shift is not trivially zero
