"""CPU oracle for decode attention over a KV cache -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never imports, links
or calls it, and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, two-pass softmax; see
its header for the passages of the pages each function follows).  This
module only builds it with gcc and marshals numpy arrays into it.

Every function here has a pin in ``tests/test_oracle_*.py`` (printed values
of the pages, closed forms, invariants, torch's library attention on small
inputs); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# a copy of oracle.c built elsewhere, loaded instead of liboracle.so: the
# planted-mistake tests run the pins against such copies in a subprocess
_OVERRIDE = os.environ.get("ATTN_ORACLE_LIB")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def threads() -> int:
    """Threads OpenMP will use for the oracle's row loop."""
    n = os.environ.get("OMP_NUM_THREADS")
    return int(n) if n else (os.cpu_count() or 1)


def _load():
    global _lib
    if _lib is None:
        if _OVERRIDE:
            lib = C.CDLL(_OVERRIDE)
        else:
            if not os.path.exists(_LIB):
                build(force=True)
            lib = C.CDLL(_LIB)
        P, I, D = C.c_void_p, C.c_int, C.c_double
        lib.ref_kv_cell_bytes.restype = C.c_ulonglong
        lib.ref_kv_cell_bytes.argtypes = [I, I, I, I]
        lib.ref_mla_cell_bytes.restype = C.c_ulonglong
        lib.ref_mla_cell_bytes.argtypes = [I, I, I, I]
        lib.ref_gqa_decode.restype = I
        lib.ref_gqa_decode.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, D]
        lib.ref_mla_absorbed.restype = I
        lib.ref_mla_absorbed.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I,
                                         I, I, I, D]
        lib.ref_mla_explicit.restype = I
        lib.ref_mla_explicit.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I,
                                         I, I, D]
        lib.ref_kv_append.restype = I
        lib.ref_kv_append.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I]
        lib.ref_fp8_e4m3_decode.restype = D
        lib.ref_fp8_e4m3_decode.argtypes = [I]
        lib.ref_fp8_e4m3_encode.restype = I
        lib.ref_fp8_e4m3_encode.argtypes = [C.c_float]
        lib.ref_gqa_decode_fp8.restype = I
        lib.ref_gqa_decode_fp8.argtypes = [P, P, P, P, P, D, D, P, P, I, I, I, I, I, I, I, D]
        lib.ref_kv_append_fp8.restype = I
        lib.ref_kv_append_fp8.argtypes = [P, P, P, P, C.c_float, C.c_float, P, P, I, I, I, I,
                                          I, I]
        lib.ref_gqa_decode_multi.restype = I
        lib.ref_gqa_decode_multi.argtypes = [P, P, P, P, P, D, D, P, P, I, I, I, I, I, I, I, I,
                                             I, D]
        lib.ref_mla_absorbed_fp8.restype = I
        lib.ref_mla_absorbed_fp8.argtypes = [P, P, P, P, P, P, P, P, D, D, P, P, I, I, I, I, I,
                                             I, I, I, I, D]
        lib.ref_mla_absorbed_multi.restype = I
        lib.ref_mla_absorbed_multi.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I,
                                               I, I, I, I, I, D]
        lib.ref_mla_absorbed_multi_fp8.restype = I
        lib.ref_mla_absorbed_multi_fp8.argtypes = [P, P, P, P, P, P, P, P, D, D, P, P, I, I, I,
                                                   I, I, I, I, I, I, I, D]
        lib.ref_mla_output.restype = I
        lib.ref_mla_output.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I,
                                       I, I, I, D]
        lib.ref_mla_absorbed_fp8_paged_scales.restype = I
        lib.ref_mla_absorbed_fp8_paged_scales.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, I,
                                                          I, I, I, I, I, I, I, D]
        lib.ref_kv_append_mla_fp8_paged_scales.restype = I
        lib.ref_kv_append_mla_fp8_paged_scales.argtypes = [P, P, P, P, P, P, I, I, I, I, I]
        lib.ref_kv_append_mla_fp8.restype = I
        lib.ref_kv_append_mla_fp8.argtypes = [P, P, C.c_float, C.c_float, P, P, I, I, I, I, I, I]
        lib.ref_gqa_decode_fp8_paged_scales.restype = I
        lib.ref_gqa_decode_fp8_paged_scales.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I,
                                                        I, D]
        lib.ref_kv_append_fp8_paged_scales.restype = I
        lib.ref_kv_append_fp8_paged_scales.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I]
        lib.ref_merge_partials.restype = I
        lib.ref_merge_partials.argtypes = [P, P, P, P, I, I, I, I, I]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _stored(a: np.ndarray, b: int) -> np.ndarray:
    want = np.uint16 if b == 2 else np.float32
    if a.dtype != want:
        raise TypeError(f"expected stored dtype {want} for b={b}, got {a.dtype}")
    return np.ascontiguousarray(a)


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def _check_table(block_table, n_rows, block_size, s):
    """Host-side guard: every mapped block id must be inside the pool."""
    if block_table is None:
        return
    for bi, n in enumerate(s):
        nb = (int(n) + block_size - 1) // block_size
        ids = block_table[bi, :nb]
        if nb and (ids.min() < 0 or ids.max() * block_size >= n_rows):
            raise ValueError(f"block table row {bi} maps outside the pool")


def kv_cell_bytes(L: int, h_kv: int, d_h: int, b: int) -> int:
    """Bytes per token over all layers: 2 * L * h_kv * d_h * b."""
    return int(_load().ref_kv_cell_bytes(L, h_kv, d_h, b))


def mla_cell_bytes(L: int, d_c: int, d_R: int, b: int) -> int:
    """Bytes per token over all layers for an MLA latent cache: L * (d_c + d_R) * b."""
    return int(_load().ref_mla_cell_bytes(L, d_c, d_R, b))


def gqa_decode(q, K, V, s, b, block_table=None, block_size=16, scale=None):
    """Reference decode attention (MHA / GQA / MQA).

    q [B,h,d_h]; K, V [B,s_max,h_kv,d_h] (contiguous) or
    [N_blk,block_size,h_kv,d_h] with block_table [B,max_blocks]; s [B].
    Arrays hold stored bits (uint16 bf16 or float32).  Returns (out [B,h,d_h]
    float64, lse [B,h] float64).
    """
    q, K, V = _stored(q, b), _stored(K, b), _stored(V, b)
    B, h, d_h = q.shape
    h_kv = K.shape[2]
    s = _i32(s)
    bt = _i32(block_table)
    if bt is None:
        s_max = K.shape[1]
        max_blocks, bs = 0, 0
    else:
        s_max = 0
        max_blocks, bs = bt.shape[1], block_size
        _check_table(bt, K.shape[0] * K.shape[1], bs, s)
    if scale is None:
        scale = 1.0 / np.sqrt(d_h)
    out = np.zeros((B, h, d_h), dtype=np.float64)
    lse = np.zeros((B, h), dtype=np.float64)
    rc = _load().ref_gqa_decode(_ptr(out), _ptr(lse), _ptr(q), _ptr(K), _ptr(V), _ptr(s),
                                _ptr(bt), max_blocks, bs, B, s_max, h, h_kv, d_h, b,
                                float(scale))
    if rc != 0:
        raise ValueError(f"ref_gqa_decode rejected its arguments ({rc})")
    return out, lse


def _mla_args(q_nope, q_rope, w_uk, w_uv, cache, s, b, block_table, block_size):
    q_nope, q_rope = _stored(q_nope, b), _stored(q_rope, b)
    w_uk, w_uv, cache = _stored(w_uk, b), _stored(w_uv, b), _stored(cache, b)
    B, h, d_nope = q_nope.shape
    d_R = q_rope.shape[2]
    d_c = w_uk.shape[2]
    d_v = w_uv.shape[1]
    if cache.shape[-1] != d_c + d_R:
        raise ValueError("cache row width must be d_c + d_R")
    s = _i32(s)
    bt = _i32(block_table)
    if bt is None:
        s_max, max_blocks, bs = cache.shape[1], 0, 0
    else:
        s_max, max_blocks, bs = 0, bt.shape[1], block_size
        _check_table(bt, cache.shape[0] * cache.shape[1], bs, s)
    return q_nope, q_rope, w_uk, w_uv, cache, s, bt, B, h, d_nope, d_R, d_c, d_v, s_max, \
        max_blocks, bs


def mla_absorbed(q_nope, q_rope, w_uk, w_uv, cache, s, b=2, block_table=None, block_size=16,
                 scale=None):
    """Reference MLA decode, absorbed form.  Returns (out [B,h,d_v], u_latent [B,h,d_c], lse [B,h])."""
    (q_nope, q_rope, w_uk, w_uv, cache, s, bt, B, h, d_nope, d_R, d_c, d_v, s_max, max_blocks,
     bs) = _mla_args(q_nope, q_rope, w_uk, w_uv, cache, s, b, block_table, block_size)
    if scale is None:
        scale = 1.0 / np.sqrt(d_nope + d_R)
    out = np.zeros((B, h, d_v), dtype=np.float64)
    ul = np.zeros((B, h, d_c), dtype=np.float64)
    lse = np.zeros((B, h), dtype=np.float64)
    rc = _load().ref_mla_absorbed(_ptr(out), _ptr(ul), _ptr(lse), _ptr(q_nope), _ptr(q_rope),
                                  _ptr(w_uk), _ptr(w_uv), _ptr(cache), _ptr(s), _ptr(bt),
                                  max_blocks, bs, B, s_max, h, d_c, d_R, d_nope, d_v, b,
                                  float(scale))
    if rc != 0:
        raise ValueError(f"ref_mla_absorbed rejected its arguments ({rc})")
    return out, ul, lse


def mla_absorbed_multi(q_nope, q_rope, w_uk, w_uv, cache, s, b=2, block_table=None,
                       block_size=16, scale=None):
    """Reference MLA decode of q_len new tokens per sequence, absorbed form.

    q_nope [B, q_len, h, d_nope], q_rope [B, q_len, h, d_R]; the cache already
    holds the q_len new tokens (s counts them) and position j sees the first
    s_b - q_len + 1 + j tokens.  Returns (out [B, q_len, h, d_v],
    u_latent [B, q_len, h, d_c], lse [B, q_len, h]).
    """
    if q_nope.ndim != 4 or q_rope.ndim != 4:
        raise ValueError("q_nope and q_rope must be [B, q_len, h, d]")
    B, q_len, h = q_nope.shape[:3]
    (q_nope, q_rope, w_uk, w_uv, cache, s, bt, _, _, d_nope, d_R, d_c, d_v, s_max, max_blocks,
     bs) = _mla_args(q_nope.reshape(B, q_len * h, -1), q_rope.reshape(B, q_len * h, -1), w_uk,
                     w_uv, cache, s, b, block_table, block_size)
    if scale is None:
        scale = 1.0 / np.sqrt(d_nope + d_R)
    out = np.zeros((B, q_len, h, d_v))
    ul = np.zeros((B, q_len, h, d_c))
    lse = np.zeros((B, q_len, h))
    rc = _load().ref_mla_absorbed_multi(_ptr(out), _ptr(ul), _ptr(lse), _ptr(q_nope),
                                        _ptr(q_rope), _ptr(w_uk), _ptr(w_uv), _ptr(cache),
                                        _ptr(s), _ptr(bt), max_blocks, bs, B, q_len, s_max, h,
                                        d_c, d_R, d_nope, d_v, b, float(scale))
    if rc != 0:
        raise ValueError(f"ref_mla_absorbed_multi rejected its arguments ({rc})")
    return out, ul, lse


def mla_output(q_nope, q_rope, w_uk, w_uv, w_o, cache, s, b=2, block_table=None, block_size=16,
               scale=None):
    """Reference MLA decode through the output projection W_O [d_model, h d_v].

    q_nope/q_rope [B, h, .] (one new token) or [B, q_len, h, .].  Returns
    (o [B, d_model] or [B, q_len, d_model], lse [B, h] or [B, q_len, h]).
    """
    multi = q_nope.ndim == 4
    if multi:
        B, q_len, h = q_nope.shape[:3]
    else:
        (B, h), q_len = q_nope.shape[:2], 1
    (q_nope, q_rope, w_uk, w_uv, cache, s, bt, _, _, d_nope, d_R, d_c, d_v, s_max, max_blocks,
     bs) = _mla_args(q_nope.reshape(B, q_len * h, -1), q_rope.reshape(B, q_len * h, -1), w_uk,
                     w_uv, cache, s, b, block_table, block_size)
    w_o = _stored(w_o, b)
    d_model = w_o.shape[0]
    if w_o.shape[1] != h * d_v:
        raise ValueError("w_o must be [d_model, h * d_v]")
    if scale is None:
        scale = 1.0 / np.sqrt(d_nope + d_R)
    o = np.zeros((B, q_len, d_model))
    lse = np.zeros((B, q_len, h))
    rc = _load().ref_mla_output(_ptr(o), _ptr(lse), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk),
                                _ptr(w_uv), _ptr(w_o), _ptr(cache), _ptr(s), _ptr(bt), max_blocks,
                                bs, B, q_len, s_max, h, d_c, d_R, d_nope, d_v, d_model, b,
                                float(scale))
    if rc != 0:
        raise ValueError(f"ref_mla_output rejected its arguments ({rc})")
    return (o, lse) if multi else (o[:, 0], lse[:, 0])


def mla_explicit(q_nope, q_rope, w_uk, w_uv, cache, s, b=2, block_table=None, block_size=16,
                 scale=None):
    """Reference MLA decode by explicit K/V expansion.  Returns (out [B,h,d_v], lse [B,h])."""
    (q_nope, q_rope, w_uk, w_uv, cache, s, bt, B, h, d_nope, d_R, d_c, d_v, s_max, max_blocks,
     bs) = _mla_args(q_nope, q_rope, w_uk, w_uv, cache, s, b, block_table, block_size)
    if scale is None:
        scale = 1.0 / np.sqrt(d_nope + d_R)
    out = np.zeros((B, h, d_v), dtype=np.float64)
    lse = np.zeros((B, h), dtype=np.float64)
    rc = _load().ref_mla_explicit(_ptr(out), _ptr(lse), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk),
                                  _ptr(w_uv), _ptr(cache), _ptr(s), _ptr(bt), max_blocks, bs, B,
                                  s_max, h, d_c, d_R, d_nope, d_v, b, float(scale))
    if rc != 0:
        raise ValueError(f"ref_mla_explicit rejected its arguments ({rc})")
    return out, lse


def kv_append(cache_k, cache_v, k_new, v_new, pos, b, block_table=None, block_size=16):
    """Reference append on host images (copies; inputs are not modified).

    cache_k/cache_v: [B,s_max,h_kv,d_h] or paged [N_blk,block_size,h_kv,d_h]
    (cache_v / v_new may be None for an MLA latent buffer, h_kv = 1).
    Returns the updated (cache_k, cache_v).
    """
    ck = _stored(cache_k, b).copy()
    cv = None if cache_v is None else _stored(cache_v, b).copy()
    kn = _stored(k_new, b)
    vn = None if v_new is None else _stored(v_new, b)
    B, h_kv, d_h = kn.shape
    pos = _i32(pos)
    bt = _i32(block_table)
    if bt is None:
        s_max, max_blocks, bs = ck.shape[1], 0, 0
    else:
        s_max, max_blocks, bs = 0, bt.shape[1], block_size
        _check_table(bt, ck.shape[0] * ck.shape[1], bs, [int(p) + 1 for p in pos])
    rc = _load().ref_kv_append(_ptr(ck), _ptr(cv), _ptr(kn), _ptr(vn), _ptr(pos), _ptr(bt),
                               max_blocks, bs, B, s_max, h_kv, d_h, b)
    if rc != 0:
        raise ValueError(f"ref_kv_append rejected its arguments ({rc})")
    return ck, cv


# ---------------------------------------------------------------------------
# FP8 (OCP E4M3) caches with one fp32 scale per tensor: value = code * scale.
# ---------------------------------------------------------------------------
def fp8_decode(codes) -> np.ndarray:
    """Values (float64) of E4M3 codes, elementwise, by the format's definition."""
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib.ref_fp8_e4m3_decode(i) for i in range(256)], dtype=np.float64)
    return table[c]


def fp8_encode(x) -> np.ndarray:
    """E4M3 codes of fp32 values: nearest, ties to even, saturating at +-448."""
    lib = _load()
    x = np.asarray(x, dtype=np.float32)
    flat = np.array([lib.ref_fp8_e4m3_encode(float(v)) for v in x.ravel()], dtype=np.uint8)
    return flat.reshape(x.shape)


def inv_scale(scale) -> np.float32:
    """The fp32 reciprocal both sides multiply by before encoding."""
    return np.float32(1.0) / np.float32(scale)


def gqa_decode_fp8(q, K8, V8, k_scale, v_scale, s, block_table=None, block_size=16,
                   scale=None):
    """Reference decode over FP8 K/V codes (uint8) with bf16 q (uint16 bits).

    Shapes as gqa_decode.  Returns (out [B,h,d_h] float64, lse [B,h] float64).
    """
    q = _stored(q, 2)
    K8 = np.ascontiguousarray(K8, dtype=np.uint8)
    V8 = np.ascontiguousarray(V8, dtype=np.uint8)
    B, h, d_h = q.shape
    h_kv = K8.shape[2]
    s = _i32(s)
    bt = _i32(block_table)
    if bt is None:
        s_max, max_blocks, bs = K8.shape[1], 0, 0
    else:
        s_max, max_blocks, bs = 0, bt.shape[1], block_size
        _check_table(bt, K8.shape[0] * K8.shape[1], bs, s)
    if scale is None:
        scale = 1.0 / np.sqrt(d_h)
    out = np.zeros((B, h, d_h), dtype=np.float64)
    lse = np.zeros((B, h), dtype=np.float64)
    rc = _load().ref_gqa_decode_fp8(_ptr(out), _ptr(lse), _ptr(q), _ptr(K8), _ptr(V8),
                                    float(np.float32(k_scale)), float(np.float32(v_scale)),
                                    _ptr(s), _ptr(bt), max_blocks, bs, B, s_max, h, h_kv, d_h,
                                    float(scale))
    if rc != 0:
        raise ValueError(f"ref_gqa_decode_fp8 rejected its arguments ({rc})")
    return out, lse


def kv_append_fp8(cache_k, cache_v, k_new, v_new, k_scale, v_scale, pos, block_table=None,
                  block_size=16):
    """Reference FP8 append on host images (copies): codes of k_new * (1/k_scale) etc."""
    ck = np.ascontiguousarray(cache_k, dtype=np.uint8).copy()
    cv = None if cache_v is None else np.ascontiguousarray(cache_v, dtype=np.uint8).copy()
    kn = _stored(k_new, 2)
    vn = None if v_new is None else _stored(v_new, 2)
    B, h_kv, d_h = kn.shape
    pos = _i32(pos)
    bt = _i32(block_table)
    if bt is None:
        s_max, max_blocks, bs = ck.shape[1], 0, 0
    else:
        s_max, max_blocks, bs = 0, bt.shape[1], block_size
        _check_table(bt, ck.shape[0] * ck.shape[1], bs, [int(p) + 1 for p in pos])
    rc = _load().ref_kv_append_fp8(_ptr(ck), _ptr(cv), _ptr(kn), _ptr(vn),
                                   float(inv_scale(k_scale)), float(inv_scale(v_scale)),
                                   _ptr(pos), _ptr(bt), max_blocks, bs, B, s_max, h_kv, d_h)
    if rc != 0:
        raise ValueError(f"ref_kv_append_fp8 rejected its arguments ({rc})")
    return ck, cv


def merge_partials(o_parts, lse_parts, b):
    """Merge decode outputs over disjoint token slices of the same sequences.

    o_parts [n,B,h,d] stored bits (uint16 bf16 or float32), lse_parts [n,B,h]
    float32 (-inf for an empty slice).  Returns (out [B,h,d] float64, lse
    [B,h] float64): lse = ln sum_k exp(lse_k), out = sum_k exp(lse_k - lse)
    o_k ("What FlashMLA solves is not the model formula itself",
    charlestar.github.io MLA page: per-block maximum, normaliser and output,
    combined stably).
    """
    o_parts = _stored(o_parts, b)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float32)
    n, B, h, d = o_parts.shape
    if lse_parts.shape != (n, B, h):
        raise ValueError("lse_parts must be [n, B, h]")
    out = np.zeros((B, h, d), dtype=np.float64)
    lse = np.zeros((B, h), dtype=np.float64)
    rc = _load().ref_merge_partials(_ptr(out), _ptr(lse), _ptr(o_parts), _ptr(lse_parts),
                                    n, B, h, d, b)
    if rc != 0:
        raise ValueError(f"ref_merge_partials rejected its arguments ({rc})")
    return out, lse


def gqa_decode_multi(q, K, V, s, b, block_table=None, block_size=16, scale=None,
                     k_scale=1.0, v_scale=1.0):
    """Reference decode of q_len new tokens per sequence (causal among them).

    q [B,q_len,h,d_h]; K, V as gqa_decode (b = 2 or 4: stored bits; b = 1:
    E4M3 codes, uint8, with per-tensor scales and bf16 q).  s[b] counts the
    cached tokens including the q_len new ones; position jq sees the first
    s[b] - q_len + 1 + jq tokens.  Returns (out [B,q_len,h,d_h] float64,
    lse [B,q_len,h] float64).
    """
    q = _stored(q, 2 if b == 1 else b)
    if b == 1:
        K = np.ascontiguousarray(K, dtype=np.uint8)
        V = np.ascontiguousarray(V, dtype=np.uint8)
    else:
        K, V = _stored(K, b), _stored(V, b)
    B, q_len, h, d_h = q.shape
    h_kv = K.shape[2]
    s = _i32(s)
    bt = _i32(block_table)
    if bt is None:
        s_max, max_blocks, bs = K.shape[1], 0, 0
    else:
        s_max, max_blocks, bs = 0, bt.shape[1], block_size
        _check_table(bt, K.shape[0] * K.shape[1], bs, s)
    if scale is None:
        scale = 1.0 / np.sqrt(d_h)
    out = np.zeros((B, q_len, h, d_h), dtype=np.float64)
    lse = np.zeros((B, q_len, h), dtype=np.float64)
    rc = _load().ref_gqa_decode_multi(_ptr(out), _ptr(lse), _ptr(q), _ptr(K), _ptr(V),
                                      float(np.float32(k_scale)), float(np.float32(v_scale)),
                                      _ptr(s), _ptr(bt), max_blocks, bs, B, q_len, s_max, h,
                                      h_kv, d_h, b, float(scale))
    if rc != 0:
        raise ValueError(f"ref_gqa_decode_multi rejected its arguments ({rc})")
    return out, lse


def mla_absorbed_fp8(q_nope, q_rope, w_uk, w_uv, cache8, c_scale, r_scale, s, block_table=None,
                     block_size=16, scale=None):
    """Reference absorbed MLA decode over an FP8 latent cache.

    cache8: uint8 E4M3 codes, rows [c (d_c) | k_R (d_R)], [B,s_max,W] or
    [N_blk,block_size,W]; element = code * c_scale (latent) or * r_scale
    (rotary).  q_nope, q_rope, w_uk, w_uv: bf16 bits.  Returns (out,
    u_latent, lse) as mla_absorbed.
    """
    q_nope, q_rope, w_uk, w_uv = (_stored(x, 2) for x in (q_nope, q_rope, w_uk, w_uv))
    cache8 = np.ascontiguousarray(cache8, dtype=np.uint8)
    B, h, d_nope = q_nope.shape
    d_R = q_rope.shape[2]
    d_c = w_uk.shape[2]
    d_v = w_uv.shape[1]
    s = _i32(s)
    bt = _i32(block_table)
    if bt is None:
        s_max, max_blocks, bs = cache8.shape[1], 0, 0
    else:
        s_max, max_blocks, bs = 0, bt.shape[1], block_size
        _check_table(bt, cache8.shape[0] * cache8.shape[1], bs, s)
    if scale is None:
        scale = 1.0 / np.sqrt(d_nope + d_R)
    out = np.zeros((B, h, d_v))
    ul = np.zeros((B, h, d_c))
    lse = np.zeros((B, h))
    rc = _load().ref_mla_absorbed_fp8(_ptr(out), _ptr(ul), _ptr(lse), _ptr(q_nope), _ptr(q_rope),
                                      _ptr(w_uk), _ptr(w_uv), _ptr(cache8),
                                      float(np.float32(c_scale)), float(np.float32(r_scale)),
                                      _ptr(s), _ptr(bt), max_blocks, bs, B, s_max, h, d_c, d_R,
                                      d_nope, d_v, float(scale))
    if rc != 0:
        raise ValueError(f"ref_mla_absorbed_fp8 rejected its arguments ({rc})")
    return out, ul, lse


def mla_absorbed_multi_fp8(q_nope, q_rope, w_uk, w_uv, cache8, c_scale, r_scale, s,
                           block_table=None, block_size=16, scale=None):
    """mla_absorbed_multi over an FP8 latent cache (scales as mla_absorbed_fp8)."""
    if q_nope.ndim != 4 or q_rope.ndim != 4:
        raise ValueError("q_nope and q_rope must be [B, q_len, h, d]")
    q_nope, q_rope, w_uk, w_uv = (_stored(x, 2) for x in (q_nope, q_rope, w_uk, w_uv))
    cache8 = np.ascontiguousarray(cache8, dtype=np.uint8)
    B, q_len, h, d_nope = q_nope.shape
    d_R = q_rope.shape[3]
    d_c = w_uk.shape[2]
    d_v = w_uv.shape[1]
    s = _i32(s)
    bt = _i32(block_table)
    if bt is None:
        s_max, max_blocks, bs = cache8.shape[1], 0, 0
    else:
        s_max, max_blocks, bs = 0, bt.shape[1], block_size
        _check_table(bt, cache8.shape[0] * cache8.shape[1], bs, s)
    if scale is None:
        scale = 1.0 / np.sqrt(d_nope + d_R)
    out = np.zeros((B, q_len, h, d_v))
    ul = np.zeros((B, q_len, h, d_c))
    lse = np.zeros((B, q_len, h))
    rc = _load().ref_mla_absorbed_multi_fp8(_ptr(out), _ptr(ul), _ptr(lse), _ptr(q_nope),
                                            _ptr(q_rope), _ptr(w_uk), _ptr(w_uv), _ptr(cache8),
                                            float(np.float32(c_scale)),
                                            float(np.float32(r_scale)), _ptr(s), _ptr(bt),
                                            max_blocks, bs, B, q_len, s_max, h, d_c, d_R,
                                            d_nope, d_v, float(scale))
    if rc != 0:
        raise ValueError(f"ref_mla_absorbed_multi_fp8 rejected its arguments ({rc})")
    return out, ul, lse


def kv_append_mla_fp8(cache8, kv_new, c_scale, r_scale, pos, d_c, block_table=None,
                      block_size=16):
    """Host image of kv_cache_append_mla_fp8: returns a new uint8 cache with
    row b of kv_new (bf16 bits [B, d_c + d_R]) encoded at slot pos[b]."""
    c = np.array(cache8, dtype=np.uint8, copy=True)
    kv_new = _stored(kv_new, 2)
    B, W = kv_new.shape
    pos = _i32(pos)
    bt = _i32(block_table)
    if bt is None:
        s_max, max_blocks, bs = c.shape[1], 0, 0
    else:
        s_max, max_blocks, bs = 0, bt.shape[1], block_size
    rc = _load().ref_kv_append_mla_fp8(_ptr(c), _ptr(kv_new), inv_scale(c_scale), inv_scale(r_scale),
                                       _ptr(pos), _ptr(bt), max_blocks, bs, B, s_max, d_c, W - d_c)
    if rc != 0:
        raise ValueError(f"ref_kv_append_mla_fp8 rejected its arguments ({rc})")
    return c


def mla_absorbed_fp8_paged_scales(q_nope, q_rope, w_uk, w_uv, cache8, c_scales, r_scales, s,
                                  block_table, block_size=16, scale=None):
    """Reference absorbed MLA decode over a paged E4M3 latent pool
    [N_blk, block_size, d_c + d_R] whose pages carry their own scales
    (c_scales, r_scales float32 [N_blk]).  Returns (out, u_latent, lse)."""
    q_nope, q_rope, w_uk, w_uv = (_stored(x, 2) for x in (q_nope, q_rope, w_uk, w_uv))
    cache8 = np.ascontiguousarray(cache8, dtype=np.uint8)
    cs = np.ascontiguousarray(c_scales, dtype=np.float32)
    rs = np.ascontiguousarray(r_scales, dtype=np.float32)
    if cs.shape != (cache8.shape[0],) or rs.shape != (cache8.shape[0],):
        raise ValueError("c_scales and r_scales must be [N_blk]")
    B, h, d_nope = q_nope.shape
    d_R = q_rope.shape[2]
    d_c = w_uk.shape[2]
    d_v = w_uv.shape[1]
    s = _i32(s)
    bt = _i32(block_table)
    _check_table(bt, cache8.shape[0] * cache8.shape[1], block_size, s)
    if scale is None:
        scale = 1.0 / np.sqrt(d_nope + d_R)
    out = np.zeros((B, h, d_v))
    ul = np.zeros((B, h, d_c))
    lse = np.zeros((B, h))
    rc = _load().ref_mla_absorbed_fp8_paged_scales(_ptr(out), _ptr(ul), _ptr(lse), _ptr(q_nope),
                                                   _ptr(q_rope), _ptr(w_uk), _ptr(w_uv),
                                                   _ptr(cache8), _ptr(cs), _ptr(rs), _ptr(s),
                                                   _ptr(bt), bt.shape[1], block_size, B, h, d_c,
                                                   d_R, d_nope, d_v, float(scale))
    if rc != 0:
        raise ValueError(f"ref_mla_absorbed_fp8_paged_scales rejected its arguments ({rc})")
    return out, ul, lse


def kv_append_mla_fp8_paged_scales(cache8, kv_new, c_scales, r_scales, pos, d_c, block_table,
                                   block_size=16):
    """Host image of kv_cache_append_mla_fp8_paged_scales: a new uint8 pool
    with row b of kv_new encoded at slot pos[b] under its page's scales."""
    c = np.array(cache8, dtype=np.uint8, copy=True)
    kv_new = _stored(kv_new, 2)
    B, W = kv_new.shape
    cs = np.ascontiguousarray(c_scales, dtype=np.float32)
    rs = np.ascontiguousarray(r_scales, dtype=np.float32)
    pos = _i32(pos)
    bt = _i32(block_table)
    rc = _load().ref_kv_append_mla_fp8_paged_scales(_ptr(c), _ptr(kv_new), _ptr(cs), _ptr(rs),
                                                    _ptr(pos), _ptr(bt), bt.shape[1], block_size,
                                                    B, d_c, W - d_c)
    if rc != 0:
        raise ValueError(f"ref_kv_append_mla_fp8_paged_scales rejected its arguments ({rc})")
    return c


def gqa_decode_fp8_paged_scales(q, K8, V8, k_scales, v_scales, s, block_table, block_size=16,
                                scale=None):
    """Reference decode over a paged E4M3 cache with one scale per page and KV
    head (k_scales, v_scales float32 [N_blk, h_kv]).  Shapes as gqa_decode."""
    q = _stored(q, 2)
    K8 = np.ascontiguousarray(K8, dtype=np.uint8)
    V8 = np.ascontiguousarray(V8, dtype=np.uint8)
    ks = np.ascontiguousarray(k_scales, dtype=np.float32)
    vs = np.ascontiguousarray(v_scales, dtype=np.float32)
    B, h, d_h = q.shape
    h_kv = K8.shape[2]
    s = _i32(s)
    bt = _i32(block_table)
    _check_table(bt, K8.shape[0] * K8.shape[1], block_size, s)
    if scale is None:
        scale = 1.0 / np.sqrt(d_h)
    out = np.zeros((B, h, d_h))
    lse = np.zeros((B, h))
    rc = _load().ref_gqa_decode_fp8_paged_scales(_ptr(out), _ptr(lse), _ptr(q), _ptr(K8), _ptr(V8),
                                                 _ptr(ks), _ptr(vs), _ptr(s), _ptr(bt), bt.shape[1],
                                                 block_size, B, h, h_kv, d_h, float(scale))
    if rc != 0:
        raise ValueError(f"ref_gqa_decode_fp8_paged_scales rejected its arguments ({rc})")
    return out, lse


def kv_append_fp8_paged_scales(cache_k, cache_v, k_new, v_new, k_scales, v_scales, pos,
                               block_table, block_size=16):
    """Host image of kv_cache_append_fp8_paged_scales (new uint8 pools)."""
    ck = np.array(cache_k, dtype=np.uint8, copy=True)
    cv = np.array(cache_v, dtype=np.uint8, copy=True)
    k_new, v_new = _stored(k_new, 2), _stored(v_new, 2)
    B, h_kv, d_h = k_new.shape
    bt = _i32(block_table)
    rc = _load().ref_kv_append_fp8_paged_scales(
        _ptr(ck), _ptr(cv), _ptr(k_new), _ptr(v_new),
        _ptr(np.ascontiguousarray(k_scales, dtype=np.float32)),
        _ptr(np.ascontiguousarray(v_scales, dtype=np.float32)), _ptr(_i32(pos)), _ptr(bt),
        bt.shape[1], block_size, B, h_kv, d_h)
    if rc != 0:
        raise ValueError(f"ref_kv_append_fp8_paged_scales rejected its arguments ({rc})")
    return ck, cv
