"""GPU kv_cache_append against the oracle's append: bit-exact."""
import numpy as np
import pytest
import torch

import decode_attention_kv_attn_amd as A
import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("b", [2, 4])
def test_contiguous_append_bit_exact(b):
    B, s_max, h_kv, d_h = 5, 33, 8, 128
    sh = synth.GqaShape("t", B=B, h=h_kv, h_kv=h_kv, d_h=d_h, b=b, s=(s_max,) * B, seed=21)
    d = synth.draw_gqa(sh, device=DEV)
    kn = torch.randn(B, h_kv, d_h, device=DEV).to(d["K"].dtype)
    vn = torch.randn(B, h_kv, d_h, device=DEV).to(d["K"].dtype)
    pos = torch.tensor([0, 32, 7, 16, 31], dtype=torch.int32, device=DEV)
    refK, refV = oracle.kv_append(synth.host_bits(d["K"]), synth.host_bits(d["V"]),
                                  synth.host_bits(kn), synth.host_bits(vn), pos.cpu().numpy(), b)
    A.kv_cache_append(d["K"], d["V"], kn, vn, pos, None, 0, 16, 0, B, s_max, h_kv, d_h, b)
    torch.cuda.synchronize()
    assert np.array_equal(synth.host_bits(d["K"]), refK)
    assert np.array_equal(synth.host_bits(d["V"]), refV)


@pytest.mark.parametrize("b", [2, 4])
def test_paged_kv_append_bit_exact(b):
    # K and V rows through a shuffled block table, positions on both sides
    # of block boundaries (first and last row of a block, a fresh block)
    s = (0, 15, 16, 31, 200)
    sh = synth.GqaShape("t", B=5, h=8, h_kv=4, d_h=128, b=b, s=tuple(x + 1 for x in s),
                        paged=True, seed=24)
    d = synth.draw_gqa(sh, device=DEV)
    kn = torch.randn(5, 4, 128, device=DEV).to(d["K"].dtype)
    vn = torch.randn(5, 4, 128, device=DEV).to(d["K"].dtype)
    pos = torch.tensor(s, dtype=torch.int32, device=DEV)
    tab = d["block_table"]
    refK, refV = oracle.kv_append(synth.host_bits(d["K"]), synth.host_bits(d["V"]),
                                  synth.host_bits(kn), synth.host_bits(vn), np.array(s, np.int32),
                                  b, block_table=d["block_table_host"])
    A.kv_cache_append(d["K"], d["V"], kn, vn, pos, tab, tab.shape[1], 16, d["K"].shape[0], 5, 0,
                      4, 128, b)
    torch.cuda.synchronize()
    assert np.array_equal(synth.host_bits(d["K"]), refK)
    assert np.array_equal(synth.host_bits(d["V"]), refV)


def test_paged_mla_latent_append_bit_exact():
    s = (0, 15, 16, 300)
    sh = synth.MlaShape("t", B=4, h=16, d_c=512, d_R=64, d_nope=128, d_v=128,
                        s=tuple(x + 1 for x in s), paged=True, seed=22)
    d = synth.draw_mla(sh, device=DEV)
    pool = d["cache"]                       # [N_blk, 16, 576]
    new = torch.randn(4, 576, device=DEV).to(torch.bfloat16)
    pos = torch.tensor(s, dtype=torch.int32, device=DEV)
    tab = d["block_table"]
    ref, _ = oracle.kv_append(synth.host_bits(pool)[:, :, None, :], None,
                              synth.host_bits(new)[:, None, :], None, np.array(s, np.int32), 2,
                              block_table=d["block_table_host"])
    A.kv_cache_append(pool, None, new, None, pos, tab, tab.shape[1], 16, pool.shape[0], 4, 0, 1,
                      576, 2)
    torch.cuda.synchronize()
    assert np.array_equal(synth.host_bits(pool), ref[:, :, 0, :])


def test_out_of_range_positions_are_skipped():
    B, s_max, h_kv, d_h = 3, 8, 2, 64
    K = torch.zeros(B, s_max, h_kv, d_h, dtype=torch.bfloat16, device=DEV)
    V = torch.zeros_like(K)
    kn = torch.ones(B, h_kv, d_h, dtype=torch.bfloat16, device=DEV)
    pos = torch.tensor([-1, 8, 3], dtype=torch.int32, device=DEV)
    A.kv_cache_append(K, V, kn, kn, pos, None, 0, 16, 0, B, s_max, h_kv, d_h, 2)
    torch.cuda.synchronize()
    assert K[0].abs().sum() == 0 and K[1].abs().sum() == 0
    assert torch.all(K[2, 3] == 1) and K[2].sum() == h_kv * d_h
