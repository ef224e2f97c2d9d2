"""Test helpers: widen stored bits to float64, draw small host inputs."""
import numpy as np
import torch

import synth


def widen(a: np.ndarray) -> np.ndarray:
    """Stored bits (uint16 bf16 or float32) -> float64, exactly."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float -> bf16 bits by round-to-nearest-even (via torch's conversion)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def stored(x: np.ndarray, b: int) -> np.ndarray:
    return bf16_bits(x) if b == 2 else np.ascontiguousarray(x, dtype=np.float32)


def gqa_host(B, h, h_kv, d_h, s, b, seed, paged=False, block_size=16):
    sh = synth.GqaShape("t", B=B, h=h, h_kv=h_kv, d_h=d_h, b=b, s=tuple(s), paged=paged,
                        block_size=block_size, seed=seed)
    d = synth.draw_gqa(sh, device="cpu")
    out = dict(q=synth.host_bits(d["q"]), K=synth.host_bits(d["K"]), V=synth.host_bits(d["V"]),
               s=d["s_host"], shape=sh)
    if paged:
        out["bt"] = d["block_table_host"]
    return out


def mla_host(B, h, d_c, d_R, d_nope, d_v, s, seed, paged=False, block_size=16, q_len=1):
    sh = synth.MlaShape("t", B=B, h=h, d_c=d_c, d_R=d_R, d_nope=d_nope, d_v=d_v, s=tuple(s),
                        paged=paged, block_size=block_size, seed=seed, q_len=q_len)
    d = synth.draw_mla(sh, device="cpu")
    out = {k: synth.host_bits(d[k]) for k in ("q_nope", "q_rope", "cache", "w_uk", "w_uv")}
    out["s"] = d["s_host"]
    out["shape"] = sh
    if paged:
        out["bt"] = d["block_table_host"]
    return out


def gather_rows(pool: np.ndarray, bt: np.ndarray, s, block_size: int, s_max: int):
    """Paged pool [N_blk, bs, ...] -> contiguous [B, s_max, ...] image (zeros past s_b)."""
    B = bt.shape[0]
    img = np.zeros((B, s_max) + pool.shape[2:], dtype=pool.dtype)
    for bi in range(B):
        for t in range(int(s[bi])):
            img[bi, t] = pool[bt[bi, t // block_size], t % block_size]
    return img
