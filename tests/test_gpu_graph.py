"""The decode entry points under HIP graph capture, as a serving loop would
run them: the calls enqueue only kernels (no allocation, no memset), so a
captured graph replays them.  Each test captures once, then replays several
times with eager work and synchronisations in between, after changing the
inputs in place, and checks every replay bit for bit against an eager call
on the same inputs (same plan, same kernels)."""
import pytest
import torch

import decode_attention_kv_attn_amd as A
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def replay_and_compare(graph, eager, outs, mutate, n=4):
    for r in range(n):
        mutate(r)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        want = eager()
        torch.cuda.synchronize()
        for g, w in zip(got, want):
            assert torch.equal(g.view(torch.uint8), w.view(torch.uint8)), f"replay {r}"
        torch.randn(1 << 20, device=DEV).sum()   # unrelated eager work between replays


@pytest.mark.parametrize("merge", ["kernel", "fused"])
def test_gqa_split_context_graph(merge, monkeypatch):
    # the merge form is fixed when the call is captured; with the in-kernel
    # merge every replay leaves the arrival counters at zero for the next
    if merge == "fused":
        monkeypatch.setenv("ATTN_GQA_MERGE", "fused")
    sh = synth.GqaShape("t", B=2, h=32, h_kv=8, d_h=128, b=2, s=(9000, 300), seed=90)
    d = synth.draw_gqa(sh, device=DEV)
    out = torch.empty_like(d["q"])
    lse = torch.empty((2, 32), dtype=torch.float32, device=DEV)
    wsb = A.attn_decode_workspace_bytes(0, 2, sh.s_max, 32, 8, 128)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    s = torch.cuda.Stream()

    def call(o, l, stream):
        A.attn_decode_gqa(o, l, d["q"], d["K"], d["V"], d["s"], None, 0, 16, 0, 2, sh.s_max, 32, 8,
                          128, 2, 0.0, ws, wsb, stream)

    with torch.cuda.stream(s):
        call(out, lse, s)   # warm up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(out, lse, s)

    def eager():
        o, l = torch.empty_like(out), torch.empty_like(lse)
        call(o, l, torch.cuda.current_stream())
        return o, l

    def mutate(r):
        d["q"].copy_(torch.randn_like(d["q"], dtype=torch.float32).to(torch.bfloat16))
        d["s"].copy_(torch.tensor([9000 - 1000 * r, 300 + r], dtype=torch.int32, device=DEV))

    replay_and_compare(g, eager, [out, lse], mutate)


def test_mla_graph():
    sh = synth.MlaShape("t", B=3, h=64, d_c=512, d_R=64, d_nope=128, d_v=128, s=(2000, 40, 700),
                        seed=91)
    d = synth.draw_mla(sh, device=DEV)
    out = torch.empty((3, 64, 128), dtype=torch.bfloat16, device=DEV)
    ul = torch.empty((3, 64, 512), dtype=torch.float32, device=DEV)
    lse = torch.empty((3, 64), dtype=torch.float32, device=DEV)
    wsb = A.attn_decode_workspace_bytes(1, 3, sh.s_max, 64, 1, 512, 64)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    s = torch.cuda.Stream()

    def call(o, u, l, stream):
        A.attn_decode_mla_absorbed(o, u, l, d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"],
                                   d["cache"], d["s"], None, 0, 16, 0, 3, sh.s_max, 64, 512, 64,
                                   128, 128, 2, 0.0, ws, wsb, stream)

    with torch.cuda.stream(s):
        call(out, ul, lse, s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(out, ul, lse, s)

    def eager():
        o, u, l = torch.empty_like(out), torch.empty_like(ul), torch.empty_like(lse)
        call(o, u, l, torch.cuda.current_stream())
        return o, u, l

    def mutate(r):
        d["q_nope"].copy_(torch.randn_like(d["q_nope"], dtype=torch.float32).to(torch.bfloat16))
        d["s"].copy_(torch.tensor([2000 - 300 * r, 40 + 7 * r, 700], dtype=torch.int32, device=DEV))

    replay_and_compare(g, eager, [out, ul, lse], mutate)


def test_append_then_decode_graph():
    # one decode step of a serving loop: append the new token's K/V, then
    # attend over the grown cache, both captured in one graph
    sh = synth.GqaShape("t", B=4, h=16, h_kv=4, d_h=128, b=2, s=(100, 700, 33, 1), paged=True,
                        seed=92)
    d = synth.draw_gqa(sh, device=DEV)
    bt = d["block_table"]
    nb, mb = d["K"].shape[0], bt.shape[1]
    smax = mb * 16
    kn = torch.randn((4, 4, 128), device=DEV).to(torch.bfloat16)
    vn = torch.randn_like(kn)
    pos = torch.tensor([99, 699, 32, 0], dtype=torch.int32, device=DEV)   # last slot of each sequence
    out = torch.empty((4, 16, 128), dtype=torch.bfloat16, device=DEV)
    wsb = A.attn_decode_workspace_bytes(0, 4, smax, 16, 4, 128)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=DEV)
    s = torch.cuda.Stream()

    def step(o, stream):
        A.kv_cache_append(d["K"], d["V"], kn, vn, pos, bt, mb, 16, nb, 4, smax, 4, 128, 2, stream)
        A.attn_decode_gqa(o, None, d["q"], d["K"], d["V"], d["s"], bt, mb, 16, nb, 4, smax, 16, 4,
                          128, 2, 0.0, ws, wsb, stream)

    with torch.cuda.stream(s):
        step(out, s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(out, s)

    def eager():
        o = torch.empty_like(out)
        step(o, torch.cuda.current_stream())
        return (o,)

    def mutate(r):
        kn.copy_(torch.randn_like(kn, dtype=torch.float32).to(torch.bfloat16))
        vn.copy_(torch.randn_like(vn, dtype=torch.float32).to(torch.bfloat16))

    replay_and_compare(g, eager, [out], mutate)


def capture_and_check(call, outs, mutate):
    """Warm up on a side stream, capture call(outs...) there, then replay and
    compare against eager calls into fresh tensors."""
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call(outs, s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(outs, s)

    def eager():
        fresh = [torch.empty_like(o) for o in outs]
        call(fresh, torch.cuda.current_stream())
        return fresh

    replay_and_compare(g, eager, outs, mutate)


def mla_shape(B, h, s, q_len=1, d_model=512, seed=95):
    return synth.MlaShape("t", B=B, h=h, d_c=512, d_R=64, d_nope=128, d_v=128, s=tuple(s),
                          seed=seed, q_len=q_len, d_model=d_model)


def mutate_mla(d, lens):
    def mutate(r):
        d["q_nope"].copy_(torch.randn_like(d["q_nope"], dtype=torch.float32).to(torch.bfloat16))
        d["s"].copy_(torch.tensor([max(n - 97 * r, 0) for n in lens], dtype=torch.int32, device=DEV))
    return mutate


def test_mla_multi_token_graph():
    lens = (1500, 40)
    sh = mla_shape(2, 32, lens, q_len=3, seed=96)
    d = synth.draw_mla(sh, device=DEV)
    ws = torch.zeros(A.attn_decode_mla_multi_workspace_bytes(2, 3, 32, 512, 64), dtype=torch.uint8,
                     device=DEV)
    outs = [torch.empty((2, 3, 32, 128), dtype=torch.bfloat16, device=DEV),
            torch.empty((2, 3, 32), dtype=torch.float32, device=DEV)]

    def call(o, st):
        A.attn_decode_mla_absorbed_multi(o[0], None, o[1], d["q_nope"], d["q_rope"], d["w_uk"],
                                         d["w_uv"], d["cache"], d["s"], None, 0, 16, 0, 2, 3,
                                         sh.s_max, 32, 512, 64, 128, 128, 2, 0.0, ws, ws.numel(),
                                         st.cuda_stream)

    capture_and_check(call, outs, mutate_mla(d, lens))


@pytest.mark.parametrize("merged", [False, True])
def test_mla_output_projection_graph(merged):
    lens = (2000, 333)
    sh = mla_shape(2, 16, lens, seed=97 + merged)
    d = synth.draw_mla(sh, device=DEV)
    w_o = synth.draw_w_o(sh, device=DEV)
    w_abs = A.premerge_weights(w_o, d["w_uv"]) if merged else None
    ws = torch.zeros(A.attn_decode_mla_out_workspace_bytes(merged, 2, 1, 16, 512, 64,
                                                           0 if merged else 128, 512),
                     dtype=torch.uint8, device=DEV)
    outs = [torch.empty((2, 512), dtype=torch.bfloat16, device=DEV),
            torch.empty((2, 16), dtype=torch.float32, device=DEV)]

    def call(o, st):
        if merged:
            A.attn_decode_mla_out_premerged(o[0], o[1], d["q_nope"], d["q_rope"], d["w_uk"], w_abs,
                                            d["cache"], d["s"], None, 0, 16, 0, 2, 1, sh.s_max, 16,
                                            512, 64, 128, 512, 2, 0.0, ws, ws.numel(), st.cuda_stream)
        else:
            A.attn_decode_mla_out(o[0], o[1], d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], w_o,
                                  d["cache"], d["s"], None, 0, 16, 0, 2, 1, sh.s_max, 16, 512, 64,
                                  128, 128, 512, 2, 0.0, ws, ws.numel(), st.cuda_stream)

    capture_and_check(call, outs, mutate_mla(d, lens))


def test_mla_mha_mode_graph():
    lens = (700, 90)
    sh = mla_shape(2, 16, lens, q_len=40, seed=99)
    d = synth.draw_mla(sh, device=DEV)
    ws = torch.zeros(A.attn_decode_mla_mha_workspace_bytes(2, sh.s_max, 16), dtype=torch.uint8,
                     device=DEV)
    outs = [torch.empty((2, 40, 16, 128), dtype=torch.bfloat16, device=DEV),
            torch.empty((2, 40, 16), dtype=torch.float32, device=DEV)]

    def call(o, st):
        A.attn_decode_mla_mha(o[0], o[1], d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["cache"],
                              d["s"], None, 0, 16, 0, 2, 40, sh.s_max, 16, 512, 64, 128, 128, 2, 0.0,
                              ws, ws.numel(), st.cuda_stream)

    capture_and_check(call, outs, mutate_mla(d, lens))
