"""Seeded synthetic inputs for decode attention over a KV cache.

This module only draws and lays out random inputs; it holds none of the
attention arithmetic.  Both the CPU oracle (through the tests) and the HIP
library (through the tests and the benchmark) are fed from here, so the two
sides always see the same stored bits.

Shapes and distributions follow the workloads of the pages:
  * "MHA -> MQA -> GQA -> MLA" (mlinterviewnotes.com), section "The four
    variants, arithmetically": Llama-3-8B / Llama-3-70B / DeepSeek-V3 head
    geometry;
  * "The KV cache size formula" (mlinterviewnotes.com), the allocated-tensor
    listing under "SGLang: one cell size, one division": token-major rows
    [rows, h_kv, d_h] for K and V, one [rows, 1, d_c + d_R] latent buffer
    for MLA;
  * "MLA: why one latent can replace a multi-head KV cache"
    (charlestar.github.io), section "What a paged KV cache block holds":
    each paged token row is [c_KV | k_R].

Recipe (every value is drawn, never computed from another input):
  * q, K, V, q_nope, q_rope and the latent cache ~ N(0, 1);
  * W_UK, W_UV ~ N(0, sigma^2) with sigma = 1/sqrt(d_c);
  * bf16 tensors are drawn in fp32 and rounded to nearest-even;
  * ragged lengths s_i ~ U{lo..hi} (inclusive) and the paged block
    permutation come from numpy PCG64 seeded with the same seed;
  * tensors come from torch's generator on the target device with
    ``manual_seed(seed)`` in a fixed draw order (q, K, V; MLA: q_nope,
    q_rope, cache, W_UK, W_UV).  Values drawn on the CPU and on a GPU differ
    (different generator streams); a test always feeds one drawn set to both
    sides, copying device inputs to the host where the oracle needs them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

BLOCK_SIZE = 16  # tokens per page, the vLLM default quoted on the cache-size page


# --------------------------------------------------------------------------
# workload shapes
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class GqaShape:
    """One decode-attention layer over a K/V cache (MHA / GQA / MQA)."""
    name: str
    B: int
    h: int
    h_kv: int
    d_h: int
    b: int                      # bytes per stored element: 2 = bf16, 4 = fp32
    s: tuple                    # per-sequence lengths s_i (len B)
    paged: bool = False
    block_size: int = BLOCK_SIZE
    seed: int = 0

    @property
    def s_max(self) -> int:
        return int(max(self.s)) if len(self.s) else 0

    @property
    def g(self) -> int:
        return self.h // self.h_kv


@dataclass(frozen=True)
class MlaShape:
    """One MLA decode layer: latent cache row [c_KV (d_c) | k_R (d_R)]."""
    name: str
    B: int
    h: int
    d_c: int
    d_R: int
    d_nope: int
    d_v: int
    s: tuple
    b: int = 2
    paged: bool = False
    block_size: int = BLOCK_SIZE
    seed: int = 0
    q_len: int = 1    # new tokens per sequence; queries are [B, q_len, h, .] when > 1
    d_model: int = 5120   # hidden size the output projection maps to

    @property
    def s_max(self) -> int:
        return int(max(self.s)) if len(self.s) else 0


def ragged_lengths(B: int, lo: int, hi: int, seed: int) -> tuple:
    """s_i ~ U{lo..hi}, drawn before any tensor of the same seed."""
    rng = np.random.default_rng(seed)
    return tuple(int(x) for x in rng.integers(lo, hi, size=B, endpoint=True))


def configs() -> dict:
    """The five workloads, by name.  Sizes are the published model shapes."""
    c = {}
    c["tiny_gqa_fp32"] = GqaShape("tiny_gqa_fp32", B=2, h=8, h_kv=2, d_h=64, b=4,
                                  s=(100, 256), seed=1)
    c["llama3_8b_gqa"] = GqaShape("llama3_8b_gqa", B=64, h=32, h_kv=8, d_h=128, b=2,
                                  s=(4096,) * 64, seed=2)
    for hkv, tag in ((64, "mha"), (8, "gqa8"), (1, "mqa")):
        c[f"llama3_70b_{tag}_b16"] = GqaShape(f"llama3_70b_{tag}_b16", B=16, h=64, h_kv=hkv,
                                              d_h=128, b=2, s=(8192,) * 16, seed=3)
        c[f"llama3_70b_{tag}_b1"] = GqaShape(f"llama3_70b_{tag}_b1", B=1, h=64, h_kv=hkv,
                                             d_h=128, b=2, s=(131072,), seed=3)
    c["deepseek_v3_mla"] = MlaShape("deepseek_v3_mla", B=32, h=128, d_c=512, d_R=64,
                                    d_nope=128, d_v=128, s=(8192,) * 32, seed=4)
    s5 = ragged_lengths(128, 128, 32768, seed=5)
    c["paged_gqa8"] = GqaShape("paged_gqa8", B=128, h=64, h_kv=8, d_h=128, b=2, s=s5,
                               paged=True, seed=5)
    c["paged_mla"] = MlaShape("paged_mla", B=128, h=128, d_c=512, d_R=64, d_nope=128,
                              d_v=128, s=s5, paged=True, seed=5)
    return c


# --------------------------------------------------------------------------
# paged block tables
# --------------------------------------------------------------------------
def block_table(s: tuple, block_size: int, seed: int, max_blocks: int | None = None):
    """Shuffled paged layout.

    Sequence b needs ceil(s_b / block_size) blocks.  Physical block ids are a
    seeded permutation of 0..N_blk-1, handed out in (b, logical block) order.
    Entries past a sequence's last block are -1.  Returns (table int32
    [B, max_blocks], N_blk).
    """
    need = [(int(x) + block_size - 1) // block_size for x in s]
    n_blk = int(sum(need))
    if max_blocks is None:
        max_blocks = max(need) if need else 1
    max_blocks = max(int(max_blocks), 1)
    rng = np.random.default_rng(seed + 1_000_003)
    perm = rng.permutation(n_blk).astype(np.int32)
    tab = np.full((len(s), max_blocks), -1, dtype=np.int32)
    k = 0
    for bi, nb in enumerate(need):
        tab[bi, :nb] = perm[k:k + nb]
        k += nb
    return tab, n_blk


def identity_table(s: tuple, block_size: int, max_blocks: int | None = None):
    """Same block counts as block_table(), physical ids in order (no shuffle)."""
    need = [(int(x) + block_size - 1) // block_size for x in s]
    n_blk = int(sum(need))
    if max_blocks is None:
        max_blocks = max(need) if need else 1
    tab = np.full((len(s), max(int(max_blocks), 1)), -1, dtype=np.int32)
    k = 0
    for bi, nb in enumerate(need):
        tab[bi, :nb] = np.arange(k, k + nb, dtype=np.int32)
        k += nb
    return tab, n_blk


# --------------------------------------------------------------------------
# drawing
# --------------------------------------------------------------------------
def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device, dtype, std=1.0, chunk=1 << 26):
    """N(0, std^2) in fp32, rounded to `dtype` (RNE for bf16), drawn in chunks."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(n, dtype=dtype, device=device)
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        x = torch.randn(hi - lo, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        out[lo:hi].copy_(x)
        del x
    return out.view(*shape)


def torch_dtype(b: int):
    return {2: torch.bfloat16, 4: torch.float32}[b]


def draw_gqa(shape: GqaShape, device="cpu", seed=None):
    """Draw q [B,h,d_h], K/V caches and lengths.

    Contiguous: K, V are [B, s_max, h_kv, d_h].  Paged: K, V are pools
    [N_blk, block_size, h_kv, d_h] plus a shuffled block table.
    """
    seed = shape.seed if seed is None else seed
    dt = torch_dtype(shape.b)
    g = _gen(device, seed)
    q = _randn((shape.B, shape.h, shape.d_h), g, device, dt)
    if shape.paged:
        tab, n_blk = block_table(shape.s, shape.block_size, seed)
        rows = (n_blk, shape.block_size)
    else:
        tab, n_blk = None, 0
        rows = (shape.B, max(shape.s_max, 1))
    K = _randn(rows + (shape.h_kv, shape.d_h), g, device, dt)
    V = _randn(rows + (shape.h_kv, shape.d_h), g, device, dt)
    s = torch.tensor(shape.s, dtype=torch.int32, device=device)
    d = dict(q=q, K=K, V=V, s=s, s_host=np.asarray(shape.s, dtype=np.int32))
    if tab is not None:
        d["block_table"] = torch.from_numpy(tab).to(device)
        d["block_table_host"] = tab
        d["n_blk"] = n_blk
    return d


def fp8_codes(x: torch.Tensor, scale: float) -> torch.Tensor:
    """E4M3 codes (uint8) that a quantizer with this per-tensor scale stores
    for x: torch's float8_e4m3fn conversion of x / scale, clamped to +-448."""
    y = (x.float() / float(np.float32(scale))).clamp_(-448.0, 448.0)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


def draw_gqa_fp8(shape: GqaShape, k_scale: float, v_scale: float, device="cpu", seed=None):
    """draw_gqa with the K/V caches stored as E4M3 codes: q is bf16, K8 and
    V8 are uint8 codes of the same N(0,1) draws divided by the scales."""
    seed = shape.seed if seed is None else seed
    g = _gen(device, seed)
    q = _randn((shape.B, shape.h, shape.d_h), g, device, torch.bfloat16)
    if shape.paged:
        tab, n_blk = block_table(shape.s, shape.block_size, seed)
        rows = (n_blk, shape.block_size)
    else:
        tab, n_blk = None, 0
        rows = (shape.B, max(shape.s_max, 1))
    K8 = fp8_codes(_randn(rows + (shape.h_kv, shape.d_h), g, device, torch.float32), k_scale)
    V8 = fp8_codes(_randn(rows + (shape.h_kv, shape.d_h), g, device, torch.float32), v_scale)
    s = torch.tensor(shape.s, dtype=torch.int32, device=device)
    d = dict(q=q, K8=K8, V8=V8, s=s, s_host=np.asarray(shape.s, dtype=np.int32))
    if tab is not None:
        d["block_table"] = torch.from_numpy(tab).to(device)
        d["block_table_host"] = tab
        d["n_blk"] = n_blk
    return d


def _mla_q_shape(shape: MlaShape, d: int) -> tuple:
    # [B, h, d] for one new token, [B, q_len, h, d] for several (the same
    # draws in the same order when q_len = 1)
    if shape.q_len == 1:
        return (shape.B, shape.h, d)
    return (shape.B, shape.q_len, shape.h, d)


def draw_mla(shape: MlaShape, device="cpu", seed=None):
    """Draw q_nope [B,h,d_nope], q_rope [B,h,d_R] (with a q_len axis after B
    when q_len > 1), latent cache, W_UK, W_UV.

    W_UK is [h, d_nope, d_c] and W_UV is [h, d_v, d_c] (per-head slices of
    the up-projections, viewed (heads, head_dim, d_c)).  Cache rows are
    [c_KV | k_R] of width d_c + d_R: [B, s_max, d_c+d_R] contiguous or
    [N_blk, block_size, d_c+d_R] paged.
    """
    seed = shape.seed if seed is None else seed
    dt = torch_dtype(shape.b)
    g = _gen(device, seed)
    q_nope = _randn(_mla_q_shape(shape, shape.d_nope), g, device, dt)
    q_rope = _randn(_mla_q_shape(shape, shape.d_R), g, device, dt)
    if shape.paged:
        tab, n_blk = block_table(shape.s, shape.block_size, seed)
        rows = (n_blk, shape.block_size)
    else:
        tab, n_blk = None, 0
        rows = (shape.B, max(shape.s_max, 1))
    cache = _randn(rows + (shape.d_c + shape.d_R,), g, device, dt)
    sig = 1.0 / math.sqrt(shape.d_c)
    w_uk = _randn((shape.h, shape.d_nope, shape.d_c), g, device, dt, std=sig)
    w_uv = _randn((shape.h, shape.d_v, shape.d_c), g, device, dt, std=sig)
    s = torch.tensor(shape.s, dtype=torch.int32, device=device)
    d = dict(q_nope=q_nope, q_rope=q_rope, cache=cache, w_uk=w_uk, w_uv=w_uv, s=s,
             s_host=np.asarray(shape.s, dtype=np.int32))
    if tab is not None:
        d["block_table"] = torch.from_numpy(tab).to(device)
        d["block_table_host"] = tab
        d["n_blk"] = n_blk
    return d


def draw_w_o(shape: MlaShape, device="cpu", seed=None):
    """Output projection W_O [d_model, h d_v] (torch Linear layout: head i owns
    columns i d_v .. i d_v + d_v - 1), N(0, 1/sqrt(h d_v)), bf16."""
    seed = (shape.seed if seed is None else seed) + 7919
    g = _gen(device, seed)
    return _randn((shape.d_model, shape.h * shape.d_v), g, device, torch.bfloat16,
                  std=1.0 / math.sqrt(shape.h * shape.d_v))


def draw_mla_fp8(shape: MlaShape, c_scale: float, r_scale: float, device="cpu", seed=None):
    """draw_mla with the latent cache stored as E4M3 codes (uint8, key
    "cache8"): the same N(0,1) rows, latent part divided by c_scale and
    rotary part by r_scale before the conversion."""
    seed = shape.seed if seed is None else seed
    g = _gen(device, seed)
    q_nope = _randn(_mla_q_shape(shape, shape.d_nope), g, device, torch.bfloat16)
    q_rope = _randn(_mla_q_shape(shape, shape.d_R), g, device, torch.bfloat16)
    if shape.paged:
        tab, n_blk = block_table(shape.s, shape.block_size, seed)
        rows = (n_blk, shape.block_size)
    else:
        tab, n_blk = None, 0
        rows = (shape.B, max(shape.s_max, 1))
    lat = _randn(rows + (shape.d_c + shape.d_R,), g, device, torch.float32)
    cache8 = torch.cat([fp8_codes(lat[..., :shape.d_c], c_scale),
                        fp8_codes(lat[..., shape.d_c:], r_scale)], dim=-1).contiguous()
    del lat
    sig = 1.0 / math.sqrt(shape.d_c)
    w_uk = _randn((shape.h, shape.d_nope, shape.d_c), g, device, torch.bfloat16, std=sig)
    w_uv = _randn((shape.h, shape.d_v, shape.d_c), g, device, torch.bfloat16, std=sig)
    s = torch.tensor(shape.s, dtype=torch.int32, device=device)
    d = dict(q_nope=q_nope, q_rope=q_rope, cache8=cache8, w_uk=w_uk, w_uv=w_uv, s=s,
             s_host=np.asarray(shape.s, dtype=np.int32))
    if tab is not None:
        d["block_table"] = torch.from_numpy(tab).to(device)
        d["block_table_host"] = tab
        d["n_blk"] = n_blk
    return d


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Stored bits of a tensor as a host numpy array (bf16 -> uint16, fp32 -> float32)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.int32:
        return t.numpy()
    if t.dtype == torch.uint8:
        return t.numpy()
    raise TypeError(t.dtype)
