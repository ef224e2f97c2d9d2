#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

One step = one attention call over the whole batch for one layer (the
decode kernel plus, when the context is split, its merge kernel).  The
headline workload is the Llama-3-8B-shaped GQA layer (B=64, h=32, h_kv=8,
d_h=128, every s_i = 4096, bf16); the DeepSeek-V3-shaped absorbed MLA layer
(B=32, h=128, d_c=512, d_R=64, s=8192) is measured in the same run and
reported under "mla", together with the E4M3-cache legs ("fp8", "mla.fp8"),
the 4-token verification leg ("multi") and the context-parallel merge
("dcp").  Inputs are synthetic (seeded N(0,1)) and resident in HBM before
timing starts.

Prints ONE JSON line.  --gpus N with N > 1 is refused: the library has no
multi-GPU path, and the benchmark measures one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attn steps/s + achieved HBM GB/s (% of peak), GQA-8 and MLA, 1 GPU"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published


def gqa_alg_bytes(sh):
    """K+V of every cached token plus q and out (bytes per call)."""
    return 2 * sum(sh.s) * sh.h_kv * sh.d_h * sh.b + 2 * sh.B * sh.h * sh.d_h * sh.b


def gqa_flops(sh):
    return 4 * sh.h * sh.d_h * sum(sh.s)


def mla_alg_bytes(sh):
    """Latent rows + W_UK + W_UV + q_nope, q_rope, out (bytes per call)."""
    return (sum(sh.s) * (sh.d_c + sh.d_R) * sh.b + sh.h * (sh.d_nope + sh.d_v) * sh.d_c * sh.b
            + sh.B * sh.h * (sh.d_nope + sh.d_R + sh.d_v) * sh.b)


def mla_fp8_alg_bytes(sh):
    """As mla_alg_bytes with one byte per cached latent element."""
    return (sum(sh.s) * (sh.d_c + sh.d_R) + sh.h * (sh.d_nope + sh.d_v) * sh.d_c * 2
            + sh.B * sh.h * (sh.d_nope + sh.d_R + sh.d_v) * 2)


def mla_flops(sh):
    return (2 * sh.h * sum(sh.s) * (2 * sh.d_c + sh.d_R)
            + 2 * sh.B * sh.h * sh.d_c * (sh.d_nope + sh.d_v))


def time_calls(fn, steps, warmup, stream):
    """Run warmup calls, then time `steps` back-to-back calls with one event
    pair around all of them (the total), then `steps` more with an event
    pair around each call (per-call durations).  Events are recorded on the
    stream the kernels run on."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        fn()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in ev])
    return total_ms, per


def run_gqa(name, steps, warmup, rotate, keep=None):
    import torch
    import synth
    import decode_attention_kv_attn_amd as A
    sh = synth.configs()[name]
    dev = "cuda"
    sets = [synth.draw_gqa(sh, device=dev, seed=sh.seed + 1000 * r) for r in range(rotate)]
    out = torch.empty_like(sets[0]["q"])
    lse = torch.empty((sh.B, sh.h), dtype=torch.float32, device=dev)
    wsb = A.attn_decode_workspace_bytes(0, sh.B, sh.s_max, sh.h, sh.h_kv, sh.d_h)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    it = [0]

    def call():
        d = sets[it[0] % rotate]
        it[0] += 1
        bt = d.get("block_table")
        A.attn_decode_gqa(out, lse, d["q"], d["K"], d["V"], d["s"], bt,
                          0 if bt is None else bt.shape[1], sh.block_size,
                          0 if bt is None else d["K"].shape[0], sh.B, sh.s_max, sh.h, sh.h_kv,
                          sh.d_h, sh.b, 0.0, ws, wsb, sp)

    total_ms, per = time_calls(call, steps, warmup, stream)
    if keep is not None:
        keep.append(sets[0])
    return sh, total_ms, per


def run_gqa_fp8(name, steps, warmup, rotate, k_scale=1.0 / 64, v_scale=1.0 / 64, pages=False):
    """The GQA workload with its K/V caches stored as E4M3 codes: per-tensor
    scales, or (pages=True, paged workloads) one K and one V scale per page
    and KV head, drawn around k_scale / v_scale."""
    import torch
    import synth
    import decode_attention_kv_attn_amd as A
    sh = synth.configs()[name]
    dev = "cuda"
    sets = [synth.draw_gqa_fp8(sh, k_scale, v_scale, device=dev, seed=sh.seed + 1000 * r)
            for r in range(rotate)]
    out = torch.empty_like(sets[0]["q"])
    lse = torch.empty((sh.B, sh.h), dtype=torch.float32, device=dev)
    wsb = A.attn_decode_workspace_bytes(0, sh.B, sh.s_max, sh.h, sh.h_kv, sh.d_h)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    it = [0]
    if pages:
        if not sh.paged:
            raise ValueError(f"{name} is not a paged workload")
        g = torch.Generator(device=dev).manual_seed(sh.seed + 17)
        n_blk = sets[0]["K8"].shape[0]
        ks = (0.5 + torch.rand((n_blk, sh.h_kv), generator=g, device=dev)) * k_scale
        vs = (0.5 + torch.rand((n_blk, sh.h_kv), generator=g, device=dev)) * v_scale

    def call():
        d = sets[it[0] % rotate]
        it[0] += 1
        bt = d.get("block_table")
        if pages:
            A.attn_decode_gqa_fp8_paged_scales(out, lse, d["q"], d["K8"], d["V8"], ks, vs, d["s"], bt,
                                               bt.shape[1], sh.block_size, d["K8"].shape[0], sh.B,
                                               sh.s_max, sh.h, sh.h_kv, sh.d_h, 0.0, ws, wsb, sp)
            return
        A.attn_decode_gqa_fp8(out, lse, d["q"], d["K8"], d["V8"], k_scale, v_scale, d["s"], bt,
                              0 if bt is None else bt.shape[1], sh.block_size,
                              0 if bt is None else d["K8"].shape[0], sh.B, sh.s_max, sh.h,
                              sh.h_kv, sh.d_h, 0.0, ws, wsb, sp)

    total_ms, per = time_calls(call, steps, warmup, stream)
    return sh, total_ms, per


def run_gqa_multi(name, q_len, steps, warmup, rotate):
    """The GQA workload with q_len new tokens per sequence (bf16 cache)."""
    import torch
    import synth
    import decode_attention_kv_attn_amd as A
    sh = synth.configs()[name]
    sets = [synth.draw_gqa(sh, device="cuda", seed=sh.seed + 1000 * r) for r in range(rotate)]
    g = torch.Generator(device="cuda").manual_seed(sh.seed)
    q = torch.randn((sh.B, q_len, sh.h, sh.d_h), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty_like(q)
    lse = torch.empty((sh.B, q_len, sh.h), dtype=torch.float32, device="cuda")
    wsb = A.attn_decode_gqa_multi_workspace_bytes(sh.B, q_len, sh.s_max, sh.h, sh.h_kv, sh.d_h)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    it = [0]

    def call():
        d = sets[it[0] % rotate]
        it[0] += 1
        bt = d.get("block_table")
        A.attn_decode_gqa_multi(out, lse, q, d["K"], d["V"], d["s"], bt,
                                0 if bt is None else bt.shape[1], sh.block_size,
                                0 if bt is None else d["K"].shape[0], sh.B, q_len, sh.s_max, sh.h,
                                sh.h_kv, sh.d_h, 2, 0.0, ws, wsb, sp)

    total_ms, per = time_calls(call, steps, warmup, stream)
    return sh, total_ms, per


def gqa_multi_alg_bytes(sh, q_len):
    """K+V of every cached token once, plus q and out of every query position."""
    return 2 * sum(sh.s) * sh.h_kv * sh.d_h * sh.b + 2 * sh.B * q_len * sh.h * sh.d_h * 2


def gqa_fp8_alg_bytes(sh):
    """K+V codes (one byte each) of every cached token plus bf16 q and out."""
    return 2 * sum(sh.s) * sh.h_kv * sh.d_h + 2 * sh.B * sh.h * sh.d_h * 2


def run_merge(n, B, h, d, steps, warmup, rotate=8):
    """attn_merge_partials over n fp32 slice partials [n,B,h,d] (+ lse) into
    fp32 [B,h,d]; input sets rotate so the Infinity Cache cannot hold them."""
    import torch
    import decode_attention_kv_attn_amd as A
    g = torch.Generator(device="cuda").manual_seed(7)
    sets = [(torch.randn((n, B, h, d), generator=g, device="cuda"),
             torch.randn((n, B, h), generator=g, device="cuda") * 4) for _ in range(rotate)]
    out = torch.empty((B, h, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, h), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    it = [0]

    def call():
        o, l = sets[it[0] % rotate]
        it[0] += 1
        A.attn_merge_partials(out, lse, o, l, n, B, h, d, 4, 4, sp)

    total_ms, per = time_calls(call, steps, warmup, stream)
    alg = (n + 1) * B * h * (d + 1) * 4
    return total_ms / steps, per, alg


def run_dcp_gqa(name, n, steps, warmup):
    """One GPU's share of context-parallel decode over n GPUs: the decode of
    a 1/n token slice of every sequence, then the merge of n such partials."""
    import torch
    import synth
    import decode_attention_kv_attn_amd as A
    sh = synth.configs()[name]
    S = (sh.s_max + n - 1) // n
    g = torch.Generator(device="cuda").manual_seed(sh.seed + 31)
    q = torch.randn((sh.B, sh.h, sh.d_h), generator=g, device="cuda").to(torch.bfloat16)
    # the slice's K/V rotate over enough sets (>= 1.2 GB) that the Infinity
    # Cache cannot serve a call from the previous one
    slice_bytes = 2 * sh.B * S * sh.h_kv * sh.d_h * 2
    rot = max(1, min(32, -(-1200000000 // slice_bytes)))
    kv = [(torch.randn((sh.B, S, sh.h_kv, sh.d_h), generator=g, device="cuda").to(torch.bfloat16),
           torch.randn((sh.B, S, sh.h_kv, sh.d_h), generator=g, device="cuda").to(torch.bfloat16))
          for _ in range(rot)]
    s = torch.full((sh.B,), S, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    parts_o = torch.empty((n, sh.B, sh.h, sh.d_h), dtype=torch.bfloat16, device="cuda")
    parts_l = torch.zeros((n, sh.B, sh.h), dtype=torch.float32, device="cuda")
    lse = torch.empty((sh.B, sh.h), dtype=torch.float32, device="cuda")
    wsb = A.attn_decode_workspace_bytes(0, sh.B, S, sh.h, sh.h_kv, sh.d_h)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    it = [0]

    def call():
        # this GPU's slice writes its own row of the gathered partials; the
        # other rows stand for the slices received from the other GPUs
        K, V = kv[it[0] % rot]
        it[0] += 1
        A.attn_decode_gqa(parts_o[0], parts_l[0], q, K, V, s, None, 0, 16, 0, sh.B, S, sh.h,
                          sh.h_kv, sh.d_h, 2, 0.0, ws, wsb, sp)
        A.attn_merge_partials(out, lse, parts_o, parts_l, n, sh.B, sh.h, sh.d_h, 2, 2, sp)

    total_ms, per = time_calls(call, steps, warmup, stream)
    del kv
    torch.cuda.empty_cache()
    return sh, S, total_ms / steps, per, rot


def run_mla(name, steps, warmup, rotate, keep=None):
    import torch
    import synth
    import decode_attention_kv_attn_amd as A
    sh = synth.configs()[name]
    dev = "cuda"
    sets = [synth.draw_mla(sh, device=dev, seed=sh.seed + 1000 * r) for r in range(rotate)]
    out = torch.empty((sh.B, sh.h, sh.d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((sh.B, sh.h), dtype=torch.float32, device=dev)
    wsb = A.attn_decode_workspace_bytes(1, sh.B, sh.s_max, sh.h, 1, sh.d_c, sh.d_R)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    it = [0]

    def call():
        d = sets[it[0] % rotate]
        it[0] += 1
        bt = d.get("block_table")
        A.attn_decode_mla_absorbed(out, None, lse, d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"],
                                   d["cache"], d["s"], bt, 0 if bt is None else bt.shape[1],
                                   sh.block_size, 0 if bt is None else d["cache"].shape[0], sh.B,
                                   sh.s_max, sh.h, sh.d_c, sh.d_R, sh.d_nope, sh.d_v, 2, 0.0, ws,
                                   wsb, sp)

    total_ms, per = time_calls(call, steps, warmup, stream)
    if keep is not None:
        keep.append(sets[0])
    return sh, total_ms, per


def run_mla_multi(name, q_len, steps, warmup, rotate):
    """The MLA workload with q_len new tokens per sequence (bf16 latent cache)."""
    import dataclasses
    import torch
    import synth
    import decode_attention_kv_attn_amd as A
    sh = dataclasses.replace(synth.configs()[name], q_len=q_len)
    sets = [synth.draw_mla(sh, device="cuda", seed=sh.seed + 1000 * r) for r in range(rotate)]
    out = torch.empty((sh.B, q_len, sh.h, sh.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((sh.B, q_len, sh.h), dtype=torch.float32, device="cuda")
    wsb = A.attn_decode_mla_multi_workspace_bytes(sh.B, q_len, sh.h, sh.d_c, sh.d_R)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    it = [0]

    def call():
        d = sets[it[0] % rotate]
        it[0] += 1
        bt = d.get("block_table")
        A.attn_decode_mla_absorbed_multi(out, None, lse, d["q_nope"], d["q_rope"], d["w_uk"],
                                         d["w_uv"], d["cache"], d["s"], bt,
                                         0 if bt is None else bt.shape[1], sh.block_size,
                                         0 if bt is None else d["cache"].shape[0], sh.B, q_len,
                                         sh.s_max, sh.h, sh.d_c, sh.d_R, sh.d_nope, sh.d_v, 2,
                                         0.0, ws, wsb, sp)

    total_ms, per = time_calls(call, steps, warmup, stream)
    return sh, total_ms, per


def mla_multi_alg_bytes(sh, q_len):
    """Latent rows once, weights once, q and out of every query position."""
    return (sum(sh.s) * (sh.d_c + sh.d_R) * sh.b + sh.h * (sh.d_nope + sh.d_v) * sh.d_c * sh.b
            + sh.B * q_len * sh.h * (sh.d_nope + sh.d_R + sh.d_v) * sh.b)


def mla_multi_flops(sh, q_len):
    """Every position scores and sums over the tokens it sees."""
    seen = sum(sum(max(n - (q_len - 1 - j), 0) for j in range(q_len)) for n in sh.s)
    return (2 * sh.h * seen * (2 * sh.d_c + sh.d_R)
            + 2 * sh.B * q_len * sh.h * sh.d_c * (sh.d_nope + sh.d_v))


def run_mla_out(name, merged, steps, warmup, rotate, d_model=5120):
    """The MLA workload through the output projection W_O [d_model, h d_v]:
    deferred (heads' outputs, then W_O) or merged (W_O^i W_UV,i, built once
    before timing)."""
    import dataclasses
    import torch
    import synth
    import decode_attention_kv_attn_amd as A
    sh = dataclasses.replace(synth.configs()[name], d_model=d_model)
    sets = [synth.draw_mla(sh, device="cuda", seed=sh.seed + 1000 * r) for r in range(rotate)]
    w_o = synth.draw_w_o(sh, device="cuda")
    w_abs = A.premerge_weights(w_o, sets[0]["w_uv"]) if merged else None
    out = torch.empty((sh.B, d_model), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((sh.B, sh.h), dtype=torch.float32, device="cuda")
    wsb = A.attn_decode_mla_out_workspace_bytes(merged, sh.B, 1, sh.h, sh.d_c, sh.d_R,
                                                0 if merged else sh.d_v, d_model)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    it = [0]

    def call():
        d = sets[it[0] % rotate]
        it[0] += 1
        if merged:
            A.attn_decode_mla_out_premerged(out, lse, d["q_nope"], d["q_rope"], d["w_uk"], w_abs,
                                            d["cache"], d["s"], None, 0, 16, 0, sh.B, 1, sh.s_max,
                                            sh.h, sh.d_c, sh.d_R, sh.d_nope, d_model, 2, 0.0, ws,
                                            wsb, sp)
        else:
            A.attn_decode_mla_out(out, lse, d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], w_o,
                                  d["cache"], d["s"], None, 0, 16, 0, sh.B, 1, sh.s_max, sh.h,
                                  sh.d_c, sh.d_R, sh.d_nope, sh.d_v, d_model, 2, 0.0, ws, wsb, sp)

    total_ms, per = time_calls(call, steps, warmup, stream)
    return sh, total_ms, per


def run_mla_mode(mha, B, s, q_len, steps, warmup, h=128, seed=77):
    """One MLA layer (d_c 512, d_R 64, d_nope = d_v = 128, bf16 latent cache)
    with q_len new tokens per sequence, in MHA mode (explicit per-head K/V)
    or in the absorbed (MQA) mode."""
    import torch
    import synth
    import decode_attention_kv_attn_amd as A
    sh = synth.MlaShape("mode", B=B, h=h, d_c=512, d_R=64, d_nope=128, d_v=128,
                        s=tuple([s] * B), seed=seed, q_len=q_len)
    d = synth.draw_mla(sh, device="cuda")
    qn = d["q_nope"] if q_len > 1 else d["q_nope"][:, None]
    qr = d["q_rope"] if q_len > 1 else d["q_rope"][:, None]
    out = torch.empty((B, q_len, h, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, q_len, h), dtype=torch.float32, device="cuda")
    if mha:
        wsb = A.attn_decode_mla_mha_workspace_bytes(B, s, h)
    else:
        wsb = A.attn_decode_mla_multi_workspace_bytes(B, q_len, h, 512, 64)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def call():
        if mha:
            A.attn_decode_mla_mha(out, lse, qn, qr, d["w_uk"], d["w_uv"], d["cache"], d["s"], None,
                                  0, 16, 0, B, q_len, s, h, 512, 64, 128, 128, 2, 0.0, ws, wsb, sp)
        else:
            A.attn_decode_mla_absorbed_multi(out, None, lse, qn, qr, d["w_uk"], d["w_uv"],
                                             d["cache"], d["s"], None, 0, 16, 0, B, q_len, s, h,
                                             512, 64, 128, 128, 2, 0.0, ws, wsb, sp)

    total_ms, per = time_calls(call, steps, warmup, stream)
    del ws, d
    torch.cuda.empty_cache()
    return total_ms / steps


def mla_modes(args):
    """Absorbed (MQA) mode vs MHA mode over query-block length and context."""
    for s in (2048, 8192):
        for ql in (1, 4, 16, 64, 256, 1024):
            steps = max(3, min(args.steps, int(2000 / ql)))
            ta = run_mla_mode(False, args.modes_batch, s, ql, steps, 2)
            tm = run_mla_mode(True, args.modes_batch, s, ql, steps, 2)
            print(f"mla-mode B={args.modes_batch} s={s:5d} q_len={ql:4d}  absorbed {ta * 1e3:10.1f} us"
                  f"  mha {tm * 1e3:10.1f} us  faster: {'mha' if tm < ta else 'absorbed'}",
                  flush=True)


def run_mla_fp8(name, steps, warmup, rotate, c_scale=1.0 / 32, r_scale=1.0 / 32):
    """The MLA workload with its latent cache stored as E4M3 codes."""
    import torch
    import synth
    import decode_attention_kv_attn_amd as A
    sh = synth.configs()[name]
    sets = [synth.draw_mla_fp8(sh, c_scale, r_scale, device="cuda", seed=sh.seed + 1000 * r)
            for r in range(rotate)]
    out = torch.empty((sh.B, sh.h, sh.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((sh.B, sh.h), dtype=torch.float32, device="cuda")
    wsb = A.attn_decode_workspace_bytes(1, sh.B, sh.s_max, sh.h, 1, sh.d_c, sh.d_R)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    it = [0]

    def call():
        d = sets[it[0] % rotate]
        it[0] += 1
        bt = d.get("block_table")
        A.attn_decode_mla_absorbed_fp8(out, None, lse, d["q_nope"], d["q_rope"], d["w_uk"],
                                       d["w_uv"], d["cache8"], c_scale, r_scale, d["s"], bt,
                                       0 if bt is None else bt.shape[1], sh.block_size,
                                       0 if bt is None else d["cache8"].shape[0], sh.B, sh.s_max,
                                       sh.h, sh.d_c, sh.d_R, sh.d_nope, sh.d_v, 0.0, ws, wsb, sp)

    total_ms, per = time_calls(call, steps, warmup, stream)
    return sh, total_ms, per


def run_mla_fp8_pages(name, steps, warmup, c_scale=1.0 / 32, r_scale=1.0 / 32, pages=True):
    """The paged MLA workload over E4M3 pages, with one scale pair per page
    (pages=True, scales drawn around c_scale / r_scale) or per-tensor scales."""
    import torch
    import synth
    import decode_attention_kv_attn_amd as A
    sh = synth.configs()[name]
    d = synth.draw_mla_fp8(sh, c_scale, r_scale, device="cuda")
    n_blk = d["cache8"].shape[0]
    g = torch.Generator(device="cuda").manual_seed(sh.seed + 17)
    cs = (0.5 + torch.rand(n_blk, generator=g, device="cuda")) * c_scale
    rs = (0.5 + torch.rand(n_blk, generator=g, device="cuda")) * r_scale
    out = torch.empty((sh.B, sh.h, sh.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((sh.B, sh.h), dtype=torch.float32, device="cuda")
    wsb = A.attn_decode_workspace_bytes(1, sh.B, sh.s_max, sh.h, 1, sh.d_c, sh.d_R)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
    bt = d["block_table"]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def call():
        if pages:
            A.attn_decode_mla_absorbed_fp8_paged_scales(out, None, lse, d["q_nope"], d["q_rope"],
                                                        d["w_uk"], d["w_uv"], d["cache8"], cs, rs,
                                                        d["s"], bt, bt.shape[1], sh.block_size,
                                                        n_blk, sh.B, sh.s_max, sh.h, sh.d_c, sh.d_R,
                                                        sh.d_nope, sh.d_v, 0.0, ws, wsb, sp)
        else:
            A.attn_decode_mla_absorbed_fp8(out, None, lse, d["q_nope"], d["q_rope"], d["w_uk"],
                                           d["w_uv"], d["cache8"], c_scale, r_scale, d["s"], bt,
                                           bt.shape[1], sh.block_size, n_blk, sh.B, sh.s_max, sh.h,
                                           sh.d_c, sh.d_R, sh.d_nope, sh.d_v, 0.0, ws, wsb, sp)

    total_ms, per = time_calls(call, steps, warmup, stream)
    return sh, total_ms, per


def cpu_baseline_gqa(sh, d, budget_s=15.0):
    """Time the oracle (as it stands) on a bounded sample of the same inputs,
    copied from the device: the first Bs sequences of the batch (all heads,
    all s_i tokens), Bs grown until one pass takes about a tenth of budget_s
    (the whole batch when it fits), then passes repeated until about budget_s
    of CPU time.  The median pass time is scaled to the full batch."""
    import oracle
    import synth

    def run(bs):
        q = synth.host_bits(d["q"][:bs])
        K = synth.host_bits(d["K"][:bs])
        V = synth.host_bits(d["V"][:bs])
        s = d["s_host"][:bs]
        t0 = time.perf_counter()
        oracle.gqa_decode(q, K, V, s, sh.b)
        return time.perf_counter() - t0

    run(1)                                    # page-in, thread pool start
    bs, dt = 1, run(1)
    if dt < budget_s / 10 and sh.B > 1:
        bs = int(min(sh.B, max(2, budget_s / 10 / max(dt, 1e-3))))
        dt = run(bs)
    times = [dt]
    while sum(times) < budget_s and len(times) < 50:
        times.append(run(bs))
    step_s = float(np.median(times)) * sh.B / bs
    return {"value": 1.0 / step_s, "unit": "steps/s", "cores": oracle.threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{bs} of {sh.B} sequences (all {sh.h} heads x {sh.s[0]} tokens); median of "
                      f"{len(times)} passes ({sum(times):.1f} s of CPU work), scaled to the full batch"}


def cpu_baseline_mla(sh, d, budget_s=5.0):
    """The absorbed MLA oracle timed the same way on the MLA workload: the
    first sequence (all heads, all its tokens) per pass, scaled to the batch."""
    import oracle
    import synth
    args = [synth.host_bits(d[k][:1]) for k in ("q_nope", "q_rope")]
    w = [synth.host_bits(d["w_uk"]), synth.host_bits(d["w_uv"])]
    C = synth.host_bits(d["cache"][:1])
    s = d["s_host"][:1]

    def run():
        t0 = time.perf_counter()
        oracle.mla_absorbed(args[0], args[1], w[0], w[1], C, s)
        return time.perf_counter() - t0

    run()
    times = [run()]
    while sum(times) < budget_s and len(times) < 20:
        times.append(run())
    step_s = float(np.median(times)) * sh.B
    return {"value": 1.0 / step_s, "unit": "steps/s", "cores": oracle.threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"1 of {sh.B} sequences (all {sh.h} heads x {sh.s[0]} tokens); median of "
                      f"{len(times)} passes ({sum(times):.1f} s of CPU work), scaled to the full batch"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# HBM traffic of the headline kernel from rocprofv3 counter passes (FETCH_SIZE
# and WRITE_SIZE, each scaled by what the counter reads for a plain device
# copy of known size), kept in profiles/ together with a digest of the kernel
# sources they were taken on; reported only while the sources are unchanged.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gqa_mfma_llama3_8b_hbm_counters.md")


# the sources that define the headline kernel (gqa_mfma_kernel), its split
# merge and its launch plan: the counter figures hold while these are unchanged
DIGEST_SOURCES = ("api.cpp", "common.h", "gqa_decode.hip", "gqa_mfma.hip", "kernels.h", "mfma_lds.h")


def kernel_source_digest():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_attention_kv_attn_amd", "csrc")
    for f in DIGEST_SOURCES:
        h.update(f.encode())
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic():
    """(bytes per launch, digest) recorded in the counter summary, or None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            kv = dict(line.split(":", 1) for line in fh if line.startswith(("traffic_bytes_per_launch:",
                                                                             "source_digest:")))
        return float(kv["traffic_bytes_per_launch"]), kv["source_digest"].strip()
    except (OSError, KeyError, ValueError):
        return None


def stream_read_gbps(reps=10):
    """Rate of the library's read probe (the decode kernels' cache-stream
    loads with nothing computed) over a 2 GiB buffer, GB/s."""
    import torch
    import decode_attention_kv_attn_amd as A
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    sink = torch.zeros(2048, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    for _ in range(2):
        A.attn_stream_read_probe(buf, nbytes, sink, sp)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        A.attn_stream_read_probe(buf, nbytes, sink, sp)
    e1.record(stream)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del buf, sink
    torch.cuda.empty_cache()
    return nbytes / (ms * 1e-3) / 1e9


SWEEP = ["llama3_8b_gqa", "llama3_70b_mha_b16", "llama3_70b_mha_b1", "llama3_70b_gqa8_b16",
         "llama3_70b_gqa8_b1", "llama3_70b_mqa_b16", "llama3_70b_mqa_b1", "paged_gqa8",
         "deepseek_v3_mla", "paged_mla"]


def sweep(args):
    """Back-to-back call time of every named workload through the library."""
    import torch
    import synth
    fp8, ql = args.sweep_cache == "fp8", args.sweep_q_len
    only = set(args.sweep_only.split(",")) if args.sweep_only else None
    for name in SWEEP:
        if only is not None and name not in only:
            continue
        sh = synth.configs()[name]
        gqa = isinstance(sh, synth.GqaShape)
        if not gqa and ql > 1:
            if fp8:
                continue
            by = mla_multi_alg_bytes(sh, ql)
            run = lambda r: run_mla_multi(name, ql, args.steps, args.warmup, r)
        elif gqa and ql > 1:
            by = gqa_multi_alg_bytes(sh, ql)
            run = lambda r: run_gqa_multi(name, ql, args.steps, args.warmup, r)
        elif gqa and fp8:
            by = gqa_fp8_alg_bytes(sh)
            run = lambda r: run_gqa_fp8(name, args.steps, args.warmup, r)
        elif gqa:
            by = gqa_alg_bytes(sh)
            run = lambda r: run_gqa(name, args.steps, args.warmup, r)
        elif fp8:
            by = mla_fp8_alg_bytes(sh)
            run = lambda r: run_mla_fp8(name, args.steps, args.warmup, r)
        else:
            by = mla_alg_bytes(sh)
            run = lambda r: run_mla(name, args.steps, args.warmup, r)
        rot = max(1, min(16, int(np.ceil(1.2e9 / by))))   # >= 1.2 GB of inputs per rotation
        _, tot, per = run(rot)
        us = tot * 1e3 / args.steps
        print(f"{name:22s} {args.sweep_cache} q_len={ql} rotate={rot:2d}  {us:9.1f} us/call  "
              f"median {float(np.median(per)) * 1e3:9.1f} us  {by / us / 1e3:7.0f} GB/s  "
              f"frac {by / us / 1e3 / HBM_PEAK_GBPS:.3f}", flush=True)
        torch.cuda.empty_cache()


LEGS = ["llama3_70b_gqa8_b16", "llama3_70b_gqa8_b1", "llama3_70b_mqa_b16", "paged_gqa8"]


def gqa_leg(name, steps, warmup):
    """One GQA workload's call time and its roofline object.  Input sets
    rotate (>= 1.2 GB per rotation) so that the Infinity Cache cannot serve
    a call from the previous one."""
    import torch
    import synth
    sh = synth.configs()[name]
    ab = gqa_alg_bytes(sh)
    rot = max(1, min(16, int(np.ceil(1.2e9 / ab))))
    _, tot, per = run_gqa(name, steps, warmup, rotate=rot)
    torch.cuda.empty_cache()
    us = tot * 1e3 / steps
    achieved = ab / (us * 1e-6) / 1e9
    lens = np.asarray(sh.s)
    return {"workload": f"{name}: GQA decode B={sh.B} h={sh.h} h_kv={sh.h_kv} d_h={sh.d_h} "
                        f"s={int(lens.min())}..{int(lens.max())} (total {int(lens.sum())} tokens)"
                        f"{' paged, 16-token blocks' if sh.paged else ''}, bf16",
            "us_per_call": us, "median_call_us": float(np.median(per)) * 1e3,
            "rotate": rot,
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                         "alg_bytes_per_call": ab}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="llama3_8b_gqa")
    ap.add_argument("--mla-config", default="deepseek_v3_mla")
    ap.add_argument("--no-mla", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-dcp", action="store_true")
    ap.add_argument("--no-multi", action="store_true")
    ap.add_argument("--no-out", action="store_true", help="skip the MLA output-projection legs")
    ap.add_argument("--mla-modes", action="store_true",
                    help="instead of the JSON line: MLA absorbed vs MHA mode over q_len and context")
    ap.add_argument("--modes-batch", type=int, default=4)
    ap.add_argument("--q-len", type=int, default=4, help="drafted tokens in the multi-token leg")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the JSON line: one line per named workload (all GQA/MQA/MHA and "
                         "MLA shapes), with input sets rotated so the Infinity Cache cannot hold them")
    ap.add_argument("--sweep-cache", choices=["bf16", "fp8"], default="bf16",
                    help="cache format of the sweep")
    ap.add_argument("--sweep-q-len", type=int, default=1, help="new tokens per sequence in the sweep")
    ap.add_argument("--sweep-only", default="",
                    help="comma-separated workload names: sweep only these (one kernel per trace)")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the Llama-3-70B-shaped and paged GQA legs")
    ap.add_argument("--mla-q-len", type=int, default=2,
                    help="new tokens per sequence in the multi-token MLA leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run a 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import decode_attention_kv_attn_amd as A
    A.lib()
    if args.calib_copy:   # a plain copy of known size, for the counter calibration
        x = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")   # 1 GiB
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        del x, y
    if args.sweep:
        sweep(args)
        return
    if args.mla_modes:
        mla_modes(args)
        return

    kept = []
    sh, total_ms, per = run_gqa(args.config, args.steps, args.warmup, rotate=1, keep=kept)
    ms = total_ms / args.steps
    call_ms = ms   # back-to-back calls: events around the timed region, on the kernels' stream
    ab = gqa_alg_bytes(sh)
    achieved = ab / (call_ms * 1e-3) / 1e9
    traffic = None
    rt = recorded_traffic()
    if rt is not None and rt[1] == kernel_source_digest() and args.config == "llama3_8b_gqa":
        traffic = rt[0]
    rec = {
        "metric": METRIC,
        "value": 1000.0 / ms,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{sh.name}: GQA decode layer B={sh.B} h={sh.h} h_kv={sh.h_kv} "
                               f"d_h={sh.d_h} s_i={sh.s[0]} bf16 (Llama-3-8B shape)",
                   "B": sh.B, "h": sh.h, "h_kv": sh.h_kv, "d_h": sh.d_h, "s": sh.s[0]},
        "hbm_gbps": ab / (ms * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": "attention call (gqa_mfma_kernel, plus gqa_combine_kernel when the context is split)",
                     "alg_bytes_per_call": ab, "avg_call_us": call_ms * 1e3,
                     "median_call_us": float(np.median(per)) * 1e3},
    }
    try:
        sgb = stream_read_gbps()
        rec["roofline"]["stream_read_gbps"] = sgb
        rec["roofline"]["frac_of_stream"] = achieved / sgb
    except Exception as e:  # the probe reports its own failure, the line still prints
        rec["roofline"]["stream_read_error"] = str(e)[:200]
    if not args.no_mla:
        try:
            mkept = []
            msh, mtot, mper = run_mla(args.mla_config, args.steps, args.warmup, rotate=4, keep=mkept)
            mms = mtot / args.steps
            mcall = mtot / args.steps
            mab = mla_alg_bytes(msh)
            mfl = mla_flops(msh)
            gbps = mab / (mcall * 1e-3) / 1e9
            tfl = mfl / (mcall * 1e-3) / 1e12
            floor_s = max(mab / (HBM_PEAK_GBPS * 1e9), mfl / (MFMA_BF16_PEAK_TFLOPS * 1e12))
            rec["mla"] = {"workload": f"{msh.name}: MLA absorbed decode B={msh.B} h={msh.h} "
                                      f"d_c={msh.d_c} d_R={msh.d_R} s={msh.s[0]} bf16",
                          "steps_per_s": 1000.0 / mms, "ms_per_step": mms,
                          "hbm_gbps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS,
                          "mfma_tflops": tfl, "mfma_frac": tfl / MFMA_BF16_PEAK_TFLOPS,
                          "roofline_frac": floor_s / (mcall * 1e-3),
                          "alg_bytes_per_call": mab, "flops_per_call": mfl}
            if not args.no_cpu_baseline:
                rec["mla"]["cpu_baseline"] = cpu_baseline_mla(msh, mkept[0])
            del mkept
        except Exception as e:  # MLA path reports its own failure, GQA line still prints
            rec["mla"] = {"error": str(e)[:200]}
        try:   # the same MLA layer over an E4M3 latent cache
            fsh, ftot, fper = run_mla_fp8(args.mla_config, args.steps, args.warmup, rotate=7)
            fms = ftot / args.steps
            fab = mla_fp8_alg_bytes(fsh)
            ffl = mla_flops(fsh)
            floor8 = max(fab / (HBM_PEAK_GBPS * 1e9), ffl / (MFMA_BF16_PEAK_TFLOPS * 1e12))
            rec["mla"]["fp8"] = {"workload": f"{fsh.name}: latent cache as E4M3 codes (latent and "
                                             f"rotary scales), bf16 q, weights and out",
                                 "steps_per_s": 1000.0 / fms, "ms_per_step": fms,
                                 "hbm_gbps": fab / (fms * 1e-3) / 1e9,
                                 "roofline_frac": floor8 / (fms * 1e-3),
                                 "alg_bytes_per_call": fab}
        except Exception as e:
            rec["mla"]["fp8"] = {"error": str(e)[:200]}
        if not args.no_fp8:
            try:   # the paged MLA batch over E4M3 pages: per-tensor scales, then a scale pair per page
                t = {}
                for key, pages in (("per_tensor", False), ("per_page", True)):
                    psh, ptot, pper = run_mla_fp8_pages("paged_mla", args.steps, args.warmup,
                                                        pages=pages)
                    t[key] = ptot / args.steps
                    torch.cuda.empty_cache()
                pab = mla_fp8_alg_bytes(psh)
                pfl = mla_flops(psh)
                pfloor = max(pab / (HBM_PEAK_GBPS * 1e9), pfl / (MFMA_BF16_PEAK_TFLOPS * 1e12))
                rec["mla"]["fp8_pages"] = {
                    "workload": f"paged_mla: B={psh.B} ragged lengths, E4M3 latent pages, one latent "
                                f"and one rotary scale per page",
                    "us_per_call": t["per_page"] * 1e3,
                    "us_per_call_per_tensor_scales": t["per_tensor"] * 1e3,
                    "roofline_frac": pfloor / (t["per_page"] * 1e-3),
                    "alg_bytes_per_call": pab}
            except Exception as e:
                rec["mla"]["fp8_pages"] = {"error": str(e)[:200]}
        if not args.no_out and "steps_per_s" in rec["mla"]:
            try:   # the same layer through the output projection, both forms
                import decode_attention_kv_attn_amd as A
                res = {}
                for form, merged in (("deferred", False), ("merged", True)):
                    osh, otot, oper = run_mla_out(args.mla_config, merged, args.steps,
                                                  args.warmup, rotate=4)
                    ous = otot * 1e3 / args.steps
                    wbytes = (osh.d_model * osh.h * osh.d_c * 2 if merged
                              else osh.d_model * osh.h * osh.d_v * 2)
                    res[form] = {"us_per_call": ous,
                                 "median_call_us": float(np.median(oper)) * 1e3,
                                 "projection_weight_bytes": wbytes,
                                 "extra_us_vs_attention": ous - rec["mla"]["ms_per_step"] * 1e3}
                    torch.cuda.empty_cache()
                rec["mla"]["out"] = {
                    "workload": f"{osh.name} through W_O [d_model={osh.d_model}, h d_v], "
                                f"deferred (heads' outputs, then W_O) vs merged "
                                f"(W_O^i W_UV,i, [d_model, h d_c])",
                    **res,
                    "form_chosen_by_rule": ("merged" if A.attn_mla_out_form(
                        osh.B, 1, osh.h, osh.d_c, osh.d_v, osh.d_model) == 1 else "deferred")}
            except Exception as e:
                rec["mla"]["out"] = {"error": str(e)[:200]}
        if not args.no_multi and "steps_per_s" in rec["mla"]:
            try:   # the same MLA layer verifying mla_q_len new tokens per sequence in one call
                ql = args.mla_q_len
                qsh, qtot, qper = run_mla_multi(args.mla_config, ql, args.steps, args.warmup,
                                                rotate=4)
                qms = qtot / args.steps
                qab = mla_multi_alg_bytes(qsh, ql)
                qfl = mla_multi_flops(qsh, ql)
                qfloor = max(qab / (HBM_PEAK_GBPS * 1e9), qfl / (MFMA_BF16_PEAK_TFLOPS * 1e12))
                rec["mla"]["multi"] = {
                    "workload": f"{qsh.name}: {ql} new tokens per sequence (causal among them), "
                                f"bf16 latent cache",
                    "q_len": ql, "steps_per_s": 1000.0 / qms, "ms_per_step": qms,
                    "query_tokens_per_s": qsh.B * ql * 1000.0 / qms,
                    "median_call_us": float(np.median(qper)) * 1e3,
                    "alg_bytes_per_call": qab, "flops_per_call": qfl,
                    "mfma_frac": qfl / (qms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                    "roofline_frac": qfloor / (qms * 1e-3),
                    "time_vs_one_token": qms / rec["mla"]["ms_per_step"]}
            except Exception as e:
                rec["mla"]["multi"] = {"error": str(e)[:200]}
    if not args.no_fp8:
        try:   # the same workload over an E4M3 cache with per-tensor scales
            fsh, ftot, fper = run_gqa_fp8(args.config, args.steps, args.warmup, rotate=2)
            fms = ftot / args.steps
            fab = gqa_fp8_alg_bytes(fsh)
            fgb = fab / (fms * 1e-3) / 1e9
            rec["fp8"] = {"workload": f"{fsh.name}: GQA decode layer, K/V caches as E4M3 codes "
                                      f"(per-tensor scales), bf16 q and out",
                          "steps_per_s": 1000.0 / fms, "ms_per_step": fms,
                          "hbm_gbps": fgb, "hbm_frac": fgb / HBM_PEAK_GBPS,
                          "alg_bytes_per_call": fab,
                          "median_call_us": float(np.median(fper)) * 1e3,
                          "speedup_vs_bf16": ms / fms}
        except Exception as e:  # the FP8 leg reports its own failure, the line still prints
            rec["fp8"] = {"error": str(e)[:200]}
        if "ms_per_step" in rec.get("fp8", {}):
            try:   # the paged GQA-8 batch over E4M3 pages: per-tensor scales, then one per page
                t = {}
                for key, pages in (("per_tensor", False), ("per_page", True)):
                    psh, ptot, pper = run_gqa_fp8("paged_gqa8", args.steps, args.warmup, rotate=1,
                                                  pages=pages)
                    t[key] = ptot / args.steps
                    torch.cuda.empty_cache()
                pab = gqa_fp8_alg_bytes(psh)
                rec["fp8"]["pages"] = {
                    "workload": f"paged_gqa8: B={psh.B} ragged lengths, E4M3 K/V pages, one K and one V "
                                f"scale per page and KV head",
                    "us_per_call": t["per_page"] * 1e3,
                    "us_per_call_per_tensor_scales": t["per_tensor"] * 1e3,
                    "hbm_frac": pab / (t["per_page"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                    "alg_bytes_per_call": pab}
            except Exception as e:
                rec["fp8"]["pages"] = {"error": str(e)[:200]}
    if not args.no_multi:
        try:   # the same layer verifying q_len drafted tokens per sequence in one call
            qsh, qtot, qper = run_gqa_multi(args.config, args.q_len, args.steps, args.warmup, rotate=1)
            qms = qtot / args.steps
            qab = gqa_multi_alg_bytes(qsh, args.q_len)
            rec["multi"] = {"workload": f"{qsh.name}: {args.q_len} new tokens per sequence "
                                        f"(causal among them), bf16 cache",
                            "q_len": args.q_len, "steps_per_s": 1000.0 / qms, "ms_per_step": qms,
                            "query_tokens_per_s": qsh.B * args.q_len * 1000.0 / qms,
                            "hbm_gbps": qab / (qms * 1e-3) / 1e9,
                            "hbm_frac": qab / (qms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                            "alg_bytes_per_call": qab,
                            "median_call_us": float(np.median(qper)) * 1e3,
                            "time_vs_one_token": qms / ms}
        except Exception as e:  # reports its own failure, the line still prints
            rec["multi"] = {"error": str(e)[:200]}
    if not args.no_legs:
        rec["legs"] = {}
        for leg in LEGS:
            try:
                rec["legs"][leg] = gqa_leg(leg, args.steps, args.warmup)
            except Exception as e:  # each leg reports its own failure
                rec["legs"][leg] = {"error": str(e)[:200]}
    if not args.no_dcp:
        try:   # the exchange step of context-parallel decode, on one GPU
            mms_, mper, malg = run_merge(8, 32, 128, 512, args.steps, args.warmup)
            dsh, S, dms, dper, drot = run_dcp_gqa("llama3_70b_gqa8_b1", 8, args.steps, args.warmup)
            rec["dcp"] = {
                "merge": {"workload": "attn_merge_partials: 8 slices of fp32 MLA latent partials "
                                      "(B=32, h=128, d_c=512) + lse -> fp32",
                          "us_per_call": mms_ * 1e3, "median_us": float(np.median(mper)) * 1e3,
                          "alg_bytes_per_call": malg,
                          "hbm_gbps": malg / (mms_ * 1e-3) / 1e9,
                          "hbm_frac": malg / (mms_ * 1e-3) / 1e9 / HBM_PEAK_GBPS},
                "gqa_slice": {"workload": f"{dsh.name}: one GPU's 1/8 token slice (s={S}) decode "
                                          f"+ merge of 8 slice partials (slice K/V rotated over "
                                          f"{drot} sets)",
                              "us_per_step": dms * 1e3, "median_us": float(np.median(dper)) * 1e3}}
        except Exception as e:  # reports its own failure, the line still prints
            rec["dcp"] = {"error": str(e)[:200]}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_gqa(sh, kept[0], args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
