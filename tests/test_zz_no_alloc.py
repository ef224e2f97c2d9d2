"""attn_decode_gqa_noalloc (the entry point that allocates nothing) against
attn_decode_gqa with a caller workspace: bit-identical outputs, on two calls
in a row, the second with a smaller input, and against the oracle."""
import numpy as np
import pytest
import torch

import decode_attention_kv_attn_amd as A
import oracle
import synth
from tests._gpu import assert_close, assert_lse_close, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(sh, d):
    """Run the workspace entry point and the no-alloc one on the same inputs."""
    bt = d.get("block_table")
    mb = 0 if bt is None else bt.shape[1]
    nblk = 0 if bt is None else d["K"].shape[0]
    s_max = sh.s_max if bt is None else mb * sh.block_size
    ws_bytes = A.attn_decode_workspace_bytes(0, sh.B, s_max, sh.h, sh.h_kv, sh.d_h)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=DEV)   # counters start at zero
    o1 = torch.full_like(d["q"], float("nan"))
    l1 = torch.full((sh.B, sh.h), float("nan"), dtype=torch.float32, device=DEV)
    A.attn_decode_gqa(o1, l1, d["q"], d["K"], d["V"], d["s"], bt, mb, sh.block_size, nblk, sh.B,
                      s_max, sh.h, sh.h_kv, sh.d_h, sh.b, 0.0, ws, ws_bytes)
    o2 = torch.full_like(d["q"], float("nan"))
    l2 = torch.full((sh.B, sh.h), float("nan"), dtype=torch.float32, device=DEV)
    A.attn_decode_gqa_noalloc(o2, l2, d["q"], d["K"], d["V"], d["s"], bt, mb, sh.block_size, nblk,
                              sh.B, s_max, sh.h, sh.h_kv, sh.d_h, sh.b, 0.0)
    torch.cuda.synchronize()
    return ws_bytes, (o1, l1), (o2, l2)


def _check_against_oracle(sh, d, o, l):
    ref, ref_lse = oracle.gqa_decode(*(synth.host_bits(d[k]) for k in ("q", "K", "V")),
                                     d["s_host"], sh.b, block_table=d.get("block_table_host"))
    assert_close(to_f64(o), ref, sh.b, "noalloc out")
    assert_lse_close(to_f64(l), ref_lse, sh.b, "noalloc lse")


@pytest.mark.parametrize("merge", ["kernel", "fused"])
@pytest.mark.parametrize("b", [2, 4])
def test_noalloc_matches_workspace_entry_twice_second_smaller(b, merge, monkeypatch):
    if merge == "fused":   # the scratch's first 64 KiB then hold the arrival counters
        monkeypatch.setenv("ATTN_GQA_MERGE", "fused")
    # first call: split contexts (the scratch holds the partials), a ragged
    # tail, an empty sequence
    big = synth.GqaShape("t", B=3, h=16, h_kv=2, d_h=128 if b == 2 else 64, b=b,
                         s=(5000, 0, 3333), seed=81)
    d = synth.draw_gqa(big, device=DEV)
    wsb, (o1, l1), (o2, l2) = _both(big, d)
    assert wsb > 0, "the first case must use the scratch"
    assert torch.equal(o1.view(torch.int16) if b == 2 else o1.view(torch.int32),
                       o2.view(torch.int16) if b == 2 else o2.view(torch.int32))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    _check_against_oracle(big, d, o2, l2)
    # second call right after: fewer sequences, shorter contexts, another g
    small = synth.GqaShape("t", B=2, h=8, h_kv=1, d_h=128 if b == 2 else 64, b=b,
                           s=(1500, 77), seed=82)
    d2 = synth.draw_gqa(small, device=DEV)
    wsb2, (o3, l3), (o4, l4) = _both(small, d2)
    assert 0 < wsb2 < wsb
    assert torch.equal(o3.view(torch.int16) if b == 2 else o3.view(torch.int32),
                       o4.view(torch.int16) if b == 2 else o4.view(torch.int32))
    assert torch.equal(l3.view(torch.int32), l4.view(torch.int32))
    _check_against_oracle(small, d2, o4, l4)


def test_noalloc_paged_then_unsplit():
    pg = synth.GqaShape("t", B=4, h=32, h_kv=4, d_h=128, b=2, s=(700, 4100, 16, 2049), paged=True,
                        seed=83)
    d = synth.draw_gqa(pg, device=DEV)
    _, (o1, l1), (o2, l2) = _both(pg, d)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    _check_against_oracle(pg, d, o2, l2)
    # a batch that needs no split (no scratch use at all)
    un = synth.GqaShape("t", B=64, h=8, h_kv=8, d_h=64, b=2, s=(130,) * 64, seed=84)
    d2 = synth.draw_gqa(un, device=DEV)
    wsb, (o3, l3), (o4, l4) = _both(un, d2)
    assert torch.equal(o3.view(torch.int16), o4.view(torch.int16))
    assert torch.equal(l3.view(torch.int32), l4.view(torch.int32))


def test_noalloc_rejects_sizes_beyond_its_scratch():
    # B = 4096, h = 64, h_kv = 8, s_max = 65536: the split partials alone
    # exceed 64 MiB; the call is rejected before anything is enqueued
    need = A.attn_decode_workspace_bytes(0, 4096, 65536, 64, 8, 128)
    assert need > (64 << 20)
    q = torch.zeros((1, 64, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(A.AttnError) as ei:
        A.attn_decode_gqa_noalloc(q, None, q, q, q, q, None, 0, 16, 0, 4096, 65536, 64, 8, 128, 2)
    assert ei.value.code == A.ATTN_ENOTSUP
    assert "scratch" in str(ei.value)
