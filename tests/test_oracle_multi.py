"""Pins for the oracle's multi-token decode (oracle.gqa_decode_multi).

q_len new tokens per sequence are already in the cache; query position jq
sees the first s_b - q_len + 1 + jq tokens (causal among the new tokens).
Checked against:
  * torch's fp64 attention with an explicit bottom-right causal mask over
    the whole [q_len x s_b] score matrix (no oracle code involved);
  * the single-token oracle (itself pinned to torch): q_len = 1 is the same
    result, and each position jq equals a single-token decode with the
    length cut to s_b - q_len + 1 + jq, for bf16, fp32 and E4M3 caches;
  * sequences shorter than q_len: the positions that see nothing give 0 and
    -inf;
  * a paged pool through a shuffled table equals its gathered image.
An off-by-one in the visible length, a swapped position/head index or a mask
on the wrong side fails at least one of these.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._util import bf16_bits, gather_rows, widen


def draw(B, q_len, h, h_kv, d, s, b, seed):
    rng = np.random.default_rng(seed)
    s_max = max(s)
    q = rng.standard_normal((B, q_len, h, d))
    K = rng.standard_normal((B, s_max, h_kv, d))
    V = rng.standard_normal((B, s_max, h_kv, d))
    conv = bf16_bits if b == 2 else (lambda x: x.astype(np.float32))
    return conv(q), conv(K), conv(V), np.array(s, np.int32)


def torch_causal(q, K, V, s):
    q, K, V = widen(q), widen(K), widen(V)
    B, T, h, d = q.shape
    g = h // K.shape[2]
    out = np.zeros((B, T, h, d))
    lse = np.full((B, T, h), -np.inf)
    for bi in range(B):
        n = int(s[bi])
        if n == 0:
            continue
        qt = torch.from_numpy(q[bi]).permute(1, 0, 2)                       # [h,T,d]
        kt = torch.from_numpy(K[bi, :n]).permute(1, 0, 2).repeat_interleave(g, 0)  # [h,n,d]
        vt = torch.from_numpy(V[bi, :n]).permute(1, 0, 2).repeat_interleave(g, 0)
        z = torch.matmul(qt, kt.transpose(1, 2)) / np.sqrt(d)              # [h,T,n]
        pos = torch.arange(T)[:, None] + (n - T)                            # cache position of each query
        z = z.masked_fill(torch.arange(n)[None, :] > pos, -float("inf"))
        l = torch.logsumexp(z, dim=2)                                       # [h,T]
        o = torch.matmul(torch.softmax(z, dim=2).nan_to_num(0.0), vt)       # [h,T,d]
        out[bi] = o.permute(1, 0, 2).numpy()
        lse[bi] = l.permute(1, 0).numpy()
    return out, lse


@pytest.mark.parametrize("b", [2, 4])
@pytest.mark.parametrize("q_len,h,h_kv", [(2, 8, 2), (4, 8, 8), (8, 4, 1), (3, 6, 2)])
def test_matches_torch_causal_attention(b, q_len, h, h_kv):
    q, K, V, s = draw(3, q_len, h, h_kv, 32, (40, 9, 17), b, seed=q_len * 10 + h)
    out, lse = oracle.gqa_decode_multi(q, K, V, s, b)
    ro, rl = torch_causal(q, K, V, s)
    assert np.max(np.abs(out - ro)) < 1e-12
    assert np.max(np.abs(lse - rl)) < 1e-12


def test_one_position_is_the_single_token_oracle():
    q, K, V, s = draw(2, 1, 8, 2, 64, (30, 7), 2, seed=1)
    out, lse = oracle.gqa_decode_multi(q, K, V, s, 2)
    ro, rl = oracle.gqa_decode(q[:, 0], K, V, s, 2)
    assert np.array_equal(out[:, 0], ro) and np.array_equal(lse[:, 0], rl)


@pytest.mark.parametrize("b", [2, 4])
def test_each_position_is_a_truncated_single_token_decode(b):
    T = 5
    q, K, V, s = draw(2, T, 8, 2, 64, (50, 12), b, seed=2)
    out, lse = oracle.gqa_decode_multi(q, K, V, s, b)
    for jq in range(T):
        sj = s - (T - 1 - jq)
        ro, rl = oracle.gqa_decode(np.ascontiguousarray(q[:, jq]), K, V, sj, b)
        assert np.array_equal(out[:, jq], ro) and np.array_equal(lse[:, jq], rl)


def test_fp8_positions_are_truncated_fp8_decodes():
    T, ks, vs = 4, 0.03, 0.05
    rng = np.random.default_rng(3)
    q = bf16_bits(rng.standard_normal((2, T, 8, 64)))
    K8 = oracle.fp8_encode((rng.standard_normal((2, 40, 2, 64)) / ks).astype(np.float32))
    V8 = oracle.fp8_encode((rng.standard_normal((2, 40, 2, 64)) / vs).astype(np.float32))
    s = np.array([40, 6], np.int32)
    out, lse = oracle.gqa_decode_multi(q, K8, V8, s, 1, k_scale=ks, v_scale=vs)
    for jq in range(T):
        ro, rl = oracle.gqa_decode_fp8(np.ascontiguousarray(q[:, jq]), K8, V8, ks, vs,
                                       s - (T - 1 - jq))
        assert np.array_equal(out[:, jq], ro) and np.array_equal(lse[:, jq], rl)


def test_sequences_shorter_than_q_len():
    T = 4
    q, K, V, s = draw(3, T, 4, 2, 16, (2, 0, 4), 4, seed=4)
    out, lse = oracle.gqa_decode_multi(q, K, V, s, 4)
    # s = 2: positions 0, 1 see nothing; s = 0: none sees anything; s = 4: all see >= 1
    assert np.all(out[0, :2] == 0) and np.all(np.isneginf(lse[0, :2]))
    assert np.all(np.isfinite(lse[0, 2:]))
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    assert np.all(np.isfinite(lse[2]))
    ro, rl = torch_causal(q, K, V, s)
    fin = np.isfinite(rl)
    assert np.max(np.abs(out[fin] - ro[fin])) < 1e-12


def test_paged_equals_gathered():
    T = 3
    sh = synth.GqaShape("t", B=3, h=8, h_kv=2, d_h=64, b=2, s=(1, 40, 70), paged=True, seed=5)
    d = synth.draw_gqa(sh, device="cpu")
    rng = np.random.default_rng(5)
    q = bf16_bits(rng.standard_normal((3, T, 8, 64)))
    Kp, Vp = synth.host_bits(d["K"]), synth.host_bits(d["V"])
    bt, s = d["block_table_host"], d["s_host"]
    out, lse = oracle.gqa_decode_multi(q, Kp, Vp, s, 2, block_table=bt)
    Ki = gather_rows(Kp, bt, s, 16, sh.s_max)
    Vi = gather_rows(Vp, bt, s, 16, sh.s_max)
    ro, rl = oracle.gqa_decode_multi(q, Ki, Vi, s, 2)
    assert np.array_equal(out, ro) and np.array_equal(lse, rl)
