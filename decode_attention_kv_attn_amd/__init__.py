"""Python binding of libattn_decode.so, the MI355X decode-attention library.

Argument marshalling only: every function forwards to the C entry point of
the same name declared in include/attn_decode.h (torch tensors become device
pointers, None becomes NULL, the stream defaults to torch's current stream).
All the computation runs in the library's HIP kernels; there is no fallback.
If the shared library has not been built this module raises on first use.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn_decode.so")

ATTN_OK, ATTN_EINVAL, ATTN_ENOTSUP, ATTN_EWORKSPACE, ATTN_EHIP = 0, -1, -2, -3, -4

EXPORTED = (
    "attn_kv_cell_bytes",
    "attn_mla_cell_bytes",
    "attn_decode_workspace_bytes",
    "attn_last_error",
    "kv_cache_append",
    "attn_decode_gqa",
    "attn_decode_mla_absorbed",
    "attn_stream_read_probe",
    "kv_cache_append_fp8",
    "attn_decode_gqa_fp8",
    "attn_merge_partials",
    "attn_decode_gqa_multi",
    "attn_decode_gqa_multi_fp8",
    "attn_decode_gqa_multi_workspace_bytes",
    "attn_decode_mla_absorbed_fp8",
    "kv_cache_append_mla_fp8",
    "attn_decode_gqa_fp8_paged_scales",
    "kv_cache_append_fp8_paged_scales",
    "attn_decode_gqa_noalloc",
    "attn_decode_mla_absorbed_multi",
    "attn_decode_mla_absorbed_multi_fp8",
    "attn_decode_mla_multi_workspace_bytes",
    "attn_decode_mla_out",
    "attn_decode_mla_out_premerged",
    "attn_decode_mla_out_workspace_bytes",
    "attn_mla_premerge_weights",
    "attn_mla_out_form",
    "attn_decode_mla_mha",
    "attn_decode_mla_mha_workspace_bytes",
    "attn_mla_mode",
    "attn_decode_mla_absorbed_fp8_paged_scales",
    "kv_cache_append_mla_fp8_paged_scales",
)

_lib = None


class AttnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"status {code}: {msg}")
        self.code = code


def lib():
    """Load the shared library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run __graft_entry__.build() "
                              "(or python -m decode_attention_kv_attn_amd.build) first")
        L = C.CDLL(LIB_PATH)
        P, I, F, Z = C.c_void_p, C.c_int, C.c_float, C.c_size_t
        L.attn_kv_cell_bytes.restype = Z
        L.attn_kv_cell_bytes.argtypes = [I, I, I, I]
        L.attn_mla_cell_bytes.restype = Z
        L.attn_mla_cell_bytes.argtypes = [I, I, I, I]
        L.attn_decode_workspace_bytes.restype = Z
        L.attn_decode_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
        L.attn_last_error.restype = C.c_char_p
        L.attn_last_error.argtypes = []
        L.kv_cache_append.restype = I
        L.kv_cache_append.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, I, P]
        L.attn_decode_gqa.restype = I
        L.attn_decode_gqa.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, P, Z, P]
        L.attn_decode_mla_absorbed.restype = I
        L.attn_decode_mla_absorbed.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I,
                                               I, I, I, I, F, P, Z, P]
        L.attn_stream_read_probe.restype = I
        L.attn_stream_read_probe.argtypes = [P, Z, P, P]
        L.kv_cache_append_fp8.restype = I
        L.kv_cache_append_fp8.argtypes = [P, P, P, P, F, F, P, P, I, I, I, I, I, I, I, P]
        L.attn_decode_gqa_fp8.restype = I
        L.attn_decode_gqa_fp8.argtypes = [P, P, P, P, P, F, F, P, P, I, I, I, I, I, I, I, I, F,
                                          P, Z, P]
        L.attn_decode_gqa_multi.restype = I
        L.attn_decode_gqa_multi.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, F,
                                            P, Z, P]
        L.attn_decode_gqa_multi_fp8.restype = I
        L.attn_decode_gqa_multi_fp8.argtypes = [P, P, P, P, P, F, F, P, P, I, I, I, I, I, I, I,
                                                I, I, F, P, Z, P]
        L.attn_decode_gqa_multi_workspace_bytes.restype = Z
        L.attn_decode_gqa_multi_workspace_bytes.argtypes = [I, I, I, I, I, I]
        L.attn_decode_mla_absorbed_fp8.restype = I
        L.attn_decode_mla_absorbed_fp8.argtypes = [P, P, P, P, P, P, P, P, F, F, P, P, I, I, I,
                                                   I, I, I, I, I, I, I, F, P, Z, P]
        L.kv_cache_append_mla_fp8.restype = I
        L.kv_cache_append_mla_fp8.argtypes = [P, P, F, F, P, P, I, I, I, I, I, I, I, P]
        L.attn_decode_gqa_fp8_paged_scales.restype = I
        L.attn_decode_gqa_fp8_paged_scales.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I,
                                                       I, I, F, P, Z, P]
        L.kv_cache_append_fp8_paged_scales.restype = I
        L.kv_cache_append_fp8_paged_scales.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I,
                                                       P]
        L.attn_decode_gqa_noalloc.restype = I
        L.attn_decode_gqa_noalloc.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, P]
        L.attn_decode_mla_absorbed_multi.restype = I
        L.attn_decode_mla_absorbed_multi.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I,
                                                     I, I, I, I, I, I, I, I, F, P, Z, P]
        L.attn_decode_mla_absorbed_multi_fp8.restype = I
        L.attn_decode_mla_absorbed_multi_fp8.argtypes = [P, P, P, P, P, P, P, P, F, F, P, P, I,
                                                         I, I, I, I, I, I, I, I, I, I, F, P, Z,
                                                         P]
        L.attn_decode_mla_multi_workspace_bytes.restype = Z
        L.attn_decode_mla_multi_workspace_bytes.argtypes = [I, I, I, I, I]
        L.attn_decode_mla_out.restype = I
        L.attn_decode_mla_out.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I,
                                          I, I, I, I, I, F, P, Z, P]
        L.attn_decode_mla_out_premerged.restype = I
        L.attn_decode_mla_out_premerged.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I,
                                                    I, I, I, I, I, I, F, P, Z, P]
        L.attn_decode_mla_out_workspace_bytes.restype = Z
        L.attn_decode_mla_out_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
        L.attn_mla_premerge_weights.restype = I
        L.attn_mla_premerge_weights.argtypes = [P, P, P, I, I, I, I, P]
        L.attn_mla_out_form.restype = I
        L.attn_mla_out_form.argtypes = [I, I, I, I, I, I]
        L.attn_decode_mla_mha.restype = I
        L.attn_decode_mla_mha.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I,
                                          I, I, I, F, P, Z, P]
        L.attn_decode_mla_mha_workspace_bytes.restype = Z
        L.attn_decode_mla_mha_workspace_bytes.argtypes = [I, I, I]
        L.attn_mla_mode.restype = I
        L.attn_mla_mode.argtypes = [I, I]
        L.attn_decode_mla_absorbed_fp8_paged_scales.restype = I
        L.attn_decode_mla_absorbed_fp8_paged_scales.argtypes = [P, P, P, P, P, P, P, P, P, P, P,
                                                                P, I, I, I, I, I, I, I, I, I, I,
                                                                F, P, Z, P]
        L.kv_cache_append_mla_fp8_paged_scales.restype = I
        L.kv_cache_append_mla_fp8_paged_scales.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I,
                                                           P]
        L.attn_merge_partials.restype = I
        L.attn_merge_partials.argtypes = [P, P, P, P, I, I, I, I, I, I, P]
        _lib = L
    return _lib


def _p(x):
    """torch tensor / int address / None -> void*."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc):
    if rc != ATTN_OK:
        raise AttnError(rc, lib().attn_last_error().decode())
    return rc


def attn_kv_cell_bytes(L, h_kv, d_h, b):
    return int(lib().attn_kv_cell_bytes(L, h_kv, d_h, b))


def attn_mla_cell_bytes(L, d_c, d_R, b):
    return int(lib().attn_mla_cell_bytes(L, d_c, d_R, b))


def attn_decode_workspace_bytes(is_mla, B, s_max, h, h_kv, d_h_or_dc, d_R=0):
    return int(lib().attn_decode_workspace_bytes(int(is_mla), B, s_max, h, h_kv, d_h_or_dc, d_R))


def attn_last_error():
    return lib().attn_last_error().decode()


def kv_cache_append(cache_k, cache_v, k_new, v_new, pos, block_table, max_blocks, block_size,
                    num_blocks, B, s_max, h_kv, d_h, b, stream=None, check=True):
    rc = lib().kv_cache_append(_p(cache_k), _p(cache_v), _p(k_new), _p(v_new), _p(pos),
                               _p(block_table), max_blocks, block_size, num_blocks, B, s_max,
                               h_kv, d_h, b, _stream(stream))
    return _check(rc) if check else rc


def attn_decode_gqa(out, lse, q, cache_k, cache_v, s, block_table, max_blocks, block_size,
                    num_blocks, B, s_max, h, h_kv, d_h, b, scale, workspace, workspace_bytes,
                    stream=None, check=True):
    rc = lib().attn_decode_gqa(_p(out), _p(lse), _p(q), _p(cache_k), _p(cache_v), _p(s),
                               _p(block_table), max_blocks, block_size, num_blocks, B, s_max, h,
                               h_kv, d_h, b, float(scale), _p(workspace), int(workspace_bytes),
                               _stream(stream))
    return _check(rc) if check else rc


def attn_decode_gqa_noalloc(out, lse, q, cache_k, cache_v, s, block_table, max_blocks,
                            block_size, num_blocks, B, s_max, h, h_kv, d_h, b, scale=0.0,
                            stream=None):
    return _check(lib().attn_decode_gqa_noalloc(
        _p(out), _p(lse), _p(q), _p(cache_k), _p(cache_v), _p(s), _p(block_table), max_blocks,
        block_size, num_blocks, B, s_max, h, h_kv, d_h, b, scale, _stream(stream)))


def kv_cache_append_fp8(cache_k, cache_v, k_new, v_new, k_scale, v_scale, pos, block_table,
                        max_blocks, block_size, num_blocks, B, s_max, h_kv, d_h, stream=None,
                        check=True):
    rc = lib().kv_cache_append_fp8(_p(cache_k), _p(cache_v), _p(k_new), _p(v_new),
                                   float(k_scale), float(v_scale), _p(pos), _p(block_table),
                                   max_blocks, block_size, num_blocks, B, s_max, h_kv, d_h,
                                   _stream(stream))
    return _check(rc) if check else rc


def attn_decode_gqa_fp8(out, lse, q, cache_k, cache_v, k_scale, v_scale, s, block_table,
                        max_blocks, block_size, num_blocks, B, s_max, h, h_kv, d_h, scale,
                        workspace, workspace_bytes, stream=None, check=True):
    rc = lib().attn_decode_gqa_fp8(_p(out), _p(lse), _p(q), _p(cache_k), _p(cache_v),
                                   float(k_scale), float(v_scale), _p(s), _p(block_table),
                                   max_blocks, block_size, num_blocks, B, s_max, h, h_kv, d_h,
                                   float(scale), _p(workspace), int(workspace_bytes),
                                   _stream(stream))
    return _check(rc) if check else rc


def attn_decode_gqa_multi(out, lse, q, cache_k, cache_v, s, block_table, max_blocks, block_size,
                          num_blocks, B, q_len, s_max, h, h_kv, d_h, b, scale, workspace,
                          workspace_bytes, stream=None, check=True):
    rc = lib().attn_decode_gqa_multi(_p(out), _p(lse), _p(q), _p(cache_k), _p(cache_v), _p(s),
                                     _p(block_table), max_blocks, block_size, num_blocks, B,
                                     q_len, s_max, h, h_kv, d_h, b, float(scale), _p(workspace),
                                     int(workspace_bytes), _stream(stream))
    return _check(rc) if check else rc


def attn_decode_gqa_multi_fp8(out, lse, q, cache_k, cache_v, k_scale, v_scale, s, block_table,
                              max_blocks, block_size, num_blocks, B, q_len, s_max, h, h_kv, d_h,
                              scale, workspace, workspace_bytes, stream=None, check=True):
    rc = lib().attn_decode_gqa_multi_fp8(_p(out), _p(lse), _p(q), _p(cache_k), _p(cache_v),
                                         float(k_scale), float(v_scale), _p(s), _p(block_table),
                                         max_blocks, block_size, num_blocks, B, q_len, s_max, h,
                                         h_kv, d_h, float(scale), _p(workspace),
                                         int(workspace_bytes), _stream(stream))
    return _check(rc) if check else rc


def attn_decode_gqa_multi_workspace_bytes(B, q_len, s_max, h, h_kv, d_h):
    return int(lib().attn_decode_gqa_multi_workspace_bytes(B, q_len, s_max, h, h_kv, d_h))


def attn_decode_mla_absorbed_fp8(out, u_latent, lse, q_nope, q_rope, w_uk, w_uv, cache, c_scale,
                                 r_scale, s, block_table, max_blocks, block_size, num_blocks, B,
                                 s_max, h, d_c, d_R, d_nope, d_v, scale, workspace,
                                 workspace_bytes, stream=None, check=True):
    rc = lib().attn_decode_mla_absorbed_fp8(_p(out), _p(u_latent), _p(lse), _p(q_nope),
                                            _p(q_rope), _p(w_uk), _p(w_uv), _p(cache),
                                            float(c_scale), float(r_scale), _p(s),
                                            _p(block_table), max_blocks, block_size, num_blocks,
                                            B, s_max, h, d_c, d_R, d_nope, d_v, float(scale),
                                            _p(workspace), int(workspace_bytes), _stream(stream))
    return _check(rc) if check else rc


def kv_cache_append_mla_fp8(cache, kv_new, c_scale, r_scale, pos, block_table, max_blocks,
                            block_size, num_blocks, B, s_max, d_c, d_R, stream=None, check=True):
    rc = lib().kv_cache_append_mla_fp8(_p(cache), _p(kv_new), float(c_scale), float(r_scale),
                                       _p(pos), _p(block_table), max_blocks, block_size,
                                       num_blocks, B, s_max, d_c, d_R, _stream(stream))
    return _check(rc) if check else rc


def attn_decode_gqa_fp8_paged_scales(out, lse, q, cache_k, cache_v, k_scales, v_scales, s,
                                     block_table, max_blocks, block_size, num_blocks, B, s_max, h,
                                     h_kv, d_h, scale, workspace, workspace_bytes, stream=None,
                                     check=True):
    rc = lib().attn_decode_gqa_fp8_paged_scales(_p(out), _p(lse), _p(q), _p(cache_k), _p(cache_v),
                                                _p(k_scales), _p(v_scales), _p(s), _p(block_table),
                                                max_blocks, block_size, num_blocks, B, s_max, h,
                                                h_kv, d_h, float(scale), _p(workspace),
                                                int(workspace_bytes), _stream(stream))
    return _check(rc) if check else rc


def kv_cache_append_fp8_paged_scales(cache_k, cache_v, k_new, v_new, k_scales, v_scales, pos,
                                     block_table, max_blocks, block_size, num_blocks, B, s_max,
                                     h_kv, d_h, stream=None, check=True):
    rc = lib().kv_cache_append_fp8_paged_scales(_p(cache_k), _p(cache_v), _p(k_new), _p(v_new),
                                                _p(k_scales), _p(v_scales), _p(pos),
                                                _p(block_table), max_blocks, block_size,
                                                num_blocks, B, s_max, h_kv, d_h, _stream(stream))
    return _check(rc) if check else rc


def attn_merge_partials(out, lse, o_parts, lse_parts, n_parts, B, h, d, b_parts, b_out,
                        stream=None, check=True):
    rc = lib().attn_merge_partials(_p(out), _p(lse), _p(o_parts), _p(lse_parts), n_parts, B, h,
                                   d, b_parts, b_out, _stream(stream))
    return _check(rc) if check else rc


def attn_stream_read_probe(src, nbytes, sink, stream=None, check=True):
    """Measurement helper (include/attn_stream_probe.h): read nbytes of src
    with the decode kernels' cache-stream loads, computing nothing."""
    rc = lib().attn_stream_read_probe(_p(src), int(nbytes), _p(sink), _stream(stream))
    return _check(rc) if check else rc


def attn_decode_mla_absorbed(out, u_latent, lse, q_nope, q_rope, w_uk, w_uv, cache, s,
                             block_table, max_blocks, block_size, num_blocks, B, s_max, h, d_c,
                             d_R, d_nope, d_v, b, scale, workspace, workspace_bytes, stream=None,
                             check=True):
    rc = lib().attn_decode_mla_absorbed(_p(out), _p(u_latent), _p(lse), _p(q_nope), _p(q_rope),
                                        _p(w_uk), _p(w_uv), _p(cache), _p(s), _p(block_table),
                                        max_blocks, block_size, num_blocks, B, s_max, h, d_c,
                                        d_R, d_nope, d_v, b, float(scale), _p(workspace),
                                        int(workspace_bytes), _stream(stream))
    return _check(rc) if check else rc


def attn_decode_mla_absorbed_multi(out, u_latent, lse, q_nope, q_rope, w_uk, w_uv, cache, s,
                                   block_table, max_blocks, block_size, num_blocks, B, q_len,
                                   s_max, h, d_c, d_R, d_nope, d_v, b, scale, workspace,
                                   workspace_bytes, stream=None, check=True):
    rc = lib().attn_decode_mla_absorbed_multi(_p(out), _p(u_latent), _p(lse), _p(q_nope),
                                              _p(q_rope), _p(w_uk), _p(w_uv), _p(cache), _p(s),
                                              _p(block_table), max_blocks, block_size,
                                              num_blocks, B, q_len, s_max, h, d_c, d_R, d_nope,
                                              d_v, b, float(scale), _p(workspace),
                                              int(workspace_bytes), _stream(stream))
    return _check(rc) if check else rc


def attn_decode_mla_absorbed_multi_fp8(out, u_latent, lse, q_nope, q_rope, w_uk, w_uv, cache,
                                       c_scale, r_scale, s, block_table, max_blocks, block_size,
                                       num_blocks, B, q_len, s_max, h, d_c, d_R, d_nope, d_v,
                                       scale, workspace, workspace_bytes, stream=None,
                                       check=True):
    rc = lib().attn_decode_mla_absorbed_multi_fp8(_p(out), _p(u_latent), _p(lse), _p(q_nope),
                                                  _p(q_rope), _p(w_uk), _p(w_uv), _p(cache),
                                                  float(c_scale), float(r_scale), _p(s),
                                                  _p(block_table), max_blocks, block_size,
                                                  num_blocks, B, q_len, s_max, h, d_c, d_R,
                                                  d_nope, d_v, float(scale), _p(workspace),
                                                  int(workspace_bytes), _stream(stream))
    return _check(rc) if check else rc


def attn_decode_mla_multi_workspace_bytes(B, q_len, h, d_c, d_R):
    return int(lib().attn_decode_mla_multi_workspace_bytes(B, q_len, h, d_c, d_R))


def attn_decode_mla_out(out, lse, q_nope, q_rope, w_uk, w_uv, w_o, cache, s, block_table,
                        max_blocks, block_size, num_blocks, B, q_len, s_max, h, d_c, d_R, d_nope,
                        d_v, d_model, b, scale, workspace, workspace_bytes, stream=None,
                        check=True):
    rc = lib().attn_decode_mla_out(_p(out), _p(lse), _p(q_nope), _p(q_rope), _p(w_uk), _p(w_uv),
                                   _p(w_o), _p(cache), _p(s), _p(block_table), max_blocks,
                                   block_size, num_blocks, B, q_len, s_max, h, d_c, d_R, d_nope,
                                   d_v, d_model, b, float(scale), _p(workspace),
                                   int(workspace_bytes), _stream(stream))
    return _check(rc) if check else rc


def attn_decode_mla_out_premerged(out, lse, q_nope, q_rope, w_uk, w_absorbed, cache, s,
                                  block_table, max_blocks, block_size, num_blocks, B, q_len,
                                  s_max, h, d_c, d_R, d_nope, d_model, b, scale, workspace,
                                  workspace_bytes, stream=None, check=True):
    rc = lib().attn_decode_mla_out_premerged(_p(out), _p(lse), _p(q_nope), _p(q_rope), _p(w_uk),
                                             _p(w_absorbed), _p(cache), _p(s), _p(block_table),
                                             max_blocks, block_size, num_blocks, B, q_len, s_max,
                                             h, d_c, d_R, d_nope, d_model, b, float(scale),
                                             _p(workspace), int(workspace_bytes),
                                             _stream(stream))
    return _check(rc) if check else rc


def attn_decode_mla_out_workspace_bytes(premerged, B, q_len, h, d_c, d_R, d_v, d_model):
    return int(lib().attn_decode_mla_out_workspace_bytes(int(premerged), B, q_len, h, d_c, d_R,
                                                         d_v, d_model))


def attn_mla_premerge_weights(w_absorbed, w_o, w_uv, h, d_c, d_v, d_model, stream=None,
                              check=True):
    rc = lib().attn_mla_premerge_weights(_p(w_absorbed), _p(w_o), _p(w_uv), h, d_c, d_v, d_model,
                                         _stream(stream))
    return _check(rc) if check else rc


def attn_mla_out_form(B, q_len, h, d_c, d_v, d_model):
    return int(lib().attn_mla_out_form(B, q_len, h, d_c, d_v, d_model))


def attn_decode_mla_mha(out, lse, q_nope, q_rope, w_uk, w_uv, cache, s, block_table, max_blocks,
                        block_size, num_blocks, B, q_len, s_max, h, d_c, d_R, d_nope, d_v, b,
                        scale, workspace, workspace_bytes, stream=None, check=True):
    rc = lib().attn_decode_mla_mha(_p(out), _p(lse), _p(q_nope), _p(q_rope), _p(w_uk), _p(w_uv),
                                   _p(cache), _p(s), _p(block_table), max_blocks, block_size,
                                   num_blocks, B, q_len, s_max, h, d_c, d_R, d_nope, d_v, b,
                                   float(scale), _p(workspace), int(workspace_bytes),
                                   _stream(stream))
    return _check(rc) if check else rc


def attn_decode_mla_mha_workspace_bytes(B, s_max, h):
    return int(lib().attn_decode_mla_mha_workspace_bytes(B, s_max, h))


def attn_mla_mode(q_len, s):
    return int(lib().attn_mla_mode(q_len, s))


def attn_decode_mla_absorbed_fp8_paged_scales(out, u_latent, lse, q_nope, q_rope, w_uk, w_uv,
                                              cache, c_scales, r_scales, s, block_table,
                                              max_blocks, block_size, num_blocks, B, s_max, h,
                                              d_c, d_R, d_nope, d_v, scale, workspace,
                                              workspace_bytes, stream=None, check=True):
    rc = lib().attn_decode_mla_absorbed_fp8_paged_scales(
        _p(out), _p(u_latent), _p(lse), _p(q_nope), _p(q_rope), _p(w_uk), _p(w_uv), _p(cache),
        _p(c_scales), _p(r_scales), _p(s), _p(block_table), max_blocks, block_size, num_blocks,
        B, s_max, h, d_c, d_R, d_nope, d_v, float(scale), _p(workspace), int(workspace_bytes),
        _stream(stream))
    return _check(rc) if check else rc


def kv_cache_append_mla_fp8_paged_scales(cache, kv_new, c_scales, r_scales, pos, block_table,
                                         max_blocks, block_size, num_blocks, B, s_max, d_c, d_R,
                                         stream=None, check=True):
    rc = lib().kv_cache_append_mla_fp8_paged_scales(_p(cache), _p(kv_new), _p(c_scales),
                                                    _p(r_scales), _p(pos), _p(block_table),
                                                    max_blocks, block_size, num_blocks, B, s_max,
                                                    d_c, d_R, _stream(stream))
    return _check(rc) if check else rc


# ---------------------------------------------------------------------------
# Convenience wrappers over torch tensors (shape bookkeeping only; they call
# the entry points above).
# ---------------------------------------------------------------------------
class Workspace:
    """A reusable device workspace (grown on demand)."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes):
        import torch
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf, self.buf.numel()


def decode_gqa(q, K, V, s, block_table=None, block_size=16, s_max=None, scale=0.0, lse=True,
               workspace=None, out=None, stream=None):
    """q [B,h,d_h]; K,V [B,s_max,h_kv,d_h] or paged pools; s [B] int32 (device)."""
    import torch
    B, h, d_h = q.shape
    h_kv = K.shape[2]
    b = q.element_size()
    if block_table is None:
        s_max = K.shape[1] if s_max is None else s_max
        max_blocks, num_blocks = 0, 0
    else:
        max_blocks = block_table.shape[1]
        num_blocks = K.shape[0]
        s_max = max_blocks * block_size if s_max is None else s_max
    if out is None:
        out = torch.empty_like(q)
    l = torch.empty((B, h), dtype=torch.float32, device=q.device) if lse else None
    ws = workspace or Workspace(q.device)
    wb, wn = ws.get(attn_decode_workspace_bytes(0, B, s_max, h, h_kv, d_h))
    attn_decode_gqa(out, l, q, K, V, s, block_table, max_blocks, block_size, num_blocks, B, s_max,
                    h, h_kv, d_h, b, scale, wb, wn, stream)
    return out, l


def decode_gqa_fp8(q, K8, V8, k_scale, v_scale, s, block_table=None, block_size=16, s_max=None,
                   scale=0.0, lse=True, workspace=None, out=None, stream=None):
    """q [B,h,d_h] bf16; K8,V8 uint8 E4M3 codes [B,s_max,h_kv,d_h] or paged pools."""
    import torch
    B, h, d_h = q.shape
    h_kv = K8.shape[2]
    if block_table is None:
        s_max = K8.shape[1] if s_max is None else s_max
        max_blocks, num_blocks = 0, 0
    else:
        max_blocks = block_table.shape[1]
        num_blocks = K8.shape[0]
        s_max = max_blocks * block_size if s_max is None else s_max
    if out is None:
        out = torch.empty_like(q)
    l = torch.empty((B, h), dtype=torch.float32, device=q.device) if lse else None
    ws = workspace or Workspace(q.device)
    wb, wn = ws.get(attn_decode_workspace_bytes(0, B, s_max, h, h_kv, d_h))
    attn_decode_gqa_fp8(out, l, q, K8, V8, k_scale, v_scale, s, block_table, max_blocks,
                        block_size, num_blocks, B, s_max, h, h_kv, d_h, scale, wb, wn, stream)
    return out, l


def decode_mla(q_nope, q_rope, w_uk, w_uv, cache, s, block_table=None, block_size=16,
               s_max=None, scale=0.0, want_latent=True, workspace=None, stream=None,
               c_scale=None, r_scale=None):
    """Absorbed MLA decode; cache rows [c | k_R] of width d_c + d_R (bf16,
    or uint8 E4M3 codes when c_scale and r_scale are given: floats, or
    [num_blocks] fp32 device tensors of per-page scales for a paged pool)."""
    import torch
    B, h, d_nope = q_nope.shape
    d_R = q_rope.shape[2]
    d_c = w_uk.shape[2]
    d_v = w_uv.shape[1]
    if block_table is None:
        s_max = cache.shape[1] if s_max is None else s_max
        max_blocks, num_blocks = 0, 0
    else:
        max_blocks = block_table.shape[1]
        num_blocks = cache.shape[0]
        s_max = max_blocks * block_size if s_max is None else s_max
    out = torch.empty((B, h, d_v), dtype=q_nope.dtype, device=q_nope.device)
    ul = torch.empty((B, h, d_c), dtype=torch.float32, device=q_nope.device) if want_latent else None
    l = torch.empty((B, h), dtype=torch.float32, device=q_nope.device)
    ws = workspace or Workspace(q_nope.device)
    wb, wn = ws.get(attn_decode_workspace_bytes(1, B, s_max, h, 1, d_c, d_R))
    if c_scale is None:
        attn_decode_mla_absorbed(out, ul, l, q_nope, q_rope, w_uk, w_uv, cache, s, block_table,
                                 max_blocks, block_size, num_blocks, B, s_max, h, d_c, d_R,
                                 d_nope, d_v, 2, scale, wb, wn, stream)
    elif not isinstance(c_scale, (int, float)):
        attn_decode_mla_absorbed_fp8_paged_scales(out, ul, l, q_nope, q_rope, w_uk, w_uv, cache,
                                                  c_scale, r_scale, s, block_table, max_blocks,
                                                  block_size, num_blocks, B, s_max, h, d_c, d_R,
                                                  d_nope, d_v, scale, wb, wn, stream)
    else:
        attn_decode_mla_absorbed_fp8(out, ul, l, q_nope, q_rope, w_uk, w_uv, cache, c_scale,
                                     r_scale, s, block_table, max_blocks, block_size, num_blocks,
                                     B, s_max, h, d_c, d_R, d_nope, d_v, scale, wb, wn, stream)
    return out, ul, l


def decode_mla_multi(q_nope, q_rope, w_uk, w_uv, cache, s, block_table=None, block_size=16,
                     s_max=None, scale=0.0, want_latent=True, workspace=None, stream=None,
                     c_scale=None, r_scale=None):
    """Absorbed MLA decode of q_len new tokens per sequence: q_nope
    [B,q_len,h,d_nope], q_rope [B,q_len,h,d_R].  Returns (out [B,q_len,h,d_v],
    u_latent [B,q_len,h,d_c] or None, lse [B,q_len,h])."""
    import torch
    B, q_len, h, d_nope = q_nope.shape
    d_R = q_rope.shape[3]
    d_c = w_uk.shape[2]
    d_v = w_uv.shape[1]
    if block_table is None:
        s_max = cache.shape[1] if s_max is None else s_max
        max_blocks, num_blocks = 0, 0
    else:
        max_blocks = block_table.shape[1]
        num_blocks = cache.shape[0]
        s_max = max_blocks * block_size if s_max is None else s_max
    dev = q_nope.device
    out = torch.empty((B, q_len, h, d_v), dtype=q_nope.dtype, device=dev)
    ul = (torch.empty((B, q_len, h, d_c), dtype=torch.float32, device=dev) if want_latent
          else None)
    l = torch.empty((B, q_len, h), dtype=torch.float32, device=dev)
    ws = workspace or Workspace(dev)
    wb, wn = ws.get(attn_decode_mla_multi_workspace_bytes(B, q_len, h, d_c, d_R))
    if c_scale is None:
        attn_decode_mla_absorbed_multi(out, ul, l, q_nope, q_rope, w_uk, w_uv, cache, s,
                                       block_table, max_blocks, block_size, num_blocks, B, q_len,
                                       s_max, h, d_c, d_R, d_nope, d_v, 2, scale, wb, wn, stream)
    else:
        attn_decode_mla_absorbed_multi_fp8(out, ul, l, q_nope, q_rope, w_uk, w_uv, cache,
                                           c_scale, r_scale, s, block_table, max_blocks,
                                           block_size, num_blocks, B, q_len, s_max, h, d_c, d_R,
                                           d_nope, d_v, scale, wb, wn, stream)
    return out, ul, l


def decode_mla_out(q_nope, q_rope, w_uk, w_o, cache, s, w_uv=None, w_absorbed=None,
                   block_table=None, block_size=16, s_max=None, scale=0.0, workspace=None,
                   stream=None):
    """MLA decode through the output projection: q_nope [B,h,d_nope] or
    [B,q_len,h,d_nope] (likewise q_rope).  Deferred form with w_uv and w_o
    [d_model, h d_v]; merged form with w_absorbed [d_model, h d_c] (from
    premerge_weights).  Returns (out [B,(q_len,)d_model] bf16, lse)."""
    import torch
    multi = q_nope.dim() == 4
    if not multi:
        q_nope, q_rope = q_nope[:, None], q_rope[:, None]
    B, q_len, h, d_nope = q_nope.shape
    d_R = q_rope.shape[3]
    d_c = w_uk.shape[2]
    merged = w_absorbed is not None
    d_model = (w_absorbed if merged else w_o).shape[0]
    d_v = 0 if merged else w_uv.shape[1]
    if block_table is None:
        s_max = cache.shape[1] if s_max is None else s_max
        max_blocks, num_blocks = 0, 0
    else:
        max_blocks, num_blocks = block_table.shape[1], cache.shape[0]
        s_max = max_blocks * block_size if s_max is None else s_max
    dev = q_nope.device
    out = torch.empty((B, q_len, d_model), dtype=torch.bfloat16, device=dev)
    l = torch.empty((B, q_len, h), dtype=torch.float32, device=dev)
    ws = workspace or Workspace(dev)
    wb, wn = ws.get(attn_decode_mla_out_workspace_bytes(merged, B, q_len, h, d_c, d_R, d_v,
                                                        d_model))
    if merged:
        attn_decode_mla_out_premerged(out, l, q_nope, q_rope, w_uk, w_absorbed, cache, s,
                                      block_table, max_blocks, block_size, num_blocks, B, q_len,
                                      s_max, h, d_c, d_R, d_nope, d_model, 2, scale, wb, wn,
                                      stream)
    else:
        attn_decode_mla_out(out, l, q_nope, q_rope, w_uk, w_uv, w_o, cache, s, block_table,
                            max_blocks, block_size, num_blocks, B, q_len, s_max, h, d_c, d_R,
                            d_nope, d_v, d_model, 2, scale, wb, wn, stream)
    return (out, l) if multi else (out[:, 0], l[:, 0])


def decode_mla_mha(q_nope, q_rope, w_uk, w_uv, cache, s, block_table=None, block_size=16,
                   s_max=None, scale=0.0, workspace=None, stream=None):
    """MLA in MHA mode (explicit per-head K/V): q_nope [B,q_len,h,128],
    q_rope [B,q_len,h,64].  Returns (out [B,q_len,h,128] bf16, lse [B,q_len,h])."""
    import torch
    B, q_len, h, d_nope = q_nope.shape
    d_R = q_rope.shape[3]
    d_c = w_uk.shape[2]
    d_v = w_uv.shape[1]
    if block_table is None:
        s_max = cache.shape[1] if s_max is None else s_max
        max_blocks, num_blocks = 0, 0
    else:
        max_blocks, num_blocks = block_table.shape[1], cache.shape[0]
        s_max = max_blocks * block_size if s_max is None else s_max
    dev = q_nope.device
    out = torch.empty((B, q_len, h, d_v), dtype=torch.bfloat16, device=dev)
    l = torch.empty((B, q_len, h), dtype=torch.float32, device=dev)
    ws = workspace or Workspace(dev)
    wb, wn = ws.get(attn_decode_mla_mha_workspace_bytes(B, s_max, h))
    attn_decode_mla_mha(out, l, q_nope, q_rope, w_uk, w_uv, cache, s, block_table, max_blocks,
                        block_size, num_blocks, B, q_len, s_max, h, d_c, d_R, d_nope, d_v, 2,
                        scale, wb, wn, stream)
    return out, l


def premerge_weights(w_o, w_uv, stream=None):
    """W_abs [d_model, h d_c] = W_O^i W_UV[i] side by side (bf16)."""
    import torch
    h, d_v, d_c = w_uv.shape
    d_model = w_o.shape[0]
    w_abs = torch.empty((d_model, h * d_c), dtype=torch.bfloat16, device=w_o.device)
    attn_mla_premerge_weights(w_abs, w_o, w_uv, h, d_c, d_v, d_model, stream)
    return w_abs


def merge_partials(o_parts, lse_parts, out_dtype=None, lse=True, stream=None):
    """Tensor form of attn_merge_partials: o_parts [n,B,h,d] (bf16 or fp32),
    lse_parts [n,B,h] fp32 -> (out [B,h,d], lse [B,h] or None)."""
    import torch
    n, B, h, d = o_parts.shape
    if tuple(lse_parts.shape) != (n, B, h) or lse_parts.dtype != torch.float32:
        raise ValueError("lse_parts must be float32 [n, B, h]")
    out_dtype = o_parts.dtype if out_dtype is None else out_dtype
    bsz = {torch.bfloat16: 2, torch.float32: 4}
    out = torch.empty((B, h, d), dtype=out_dtype, device=o_parts.device)
    l = torch.empty((B, h), dtype=torch.float32, device=o_parts.device) if lse else None
    attn_merge_partials(out, l, o_parts.contiguous(), lse_parts.contiguous(), n, B, h, d,
                        bsz[o_parts.dtype], bsz[out_dtype], stream)
    return out, l


def decode_gqa_multi(q, K, V, s, block_table=None, block_size=16, s_max=None, scale=0.0,
                     lse=True, k_scale=None, v_scale=None, workspace=None, stream=None):
    """Decode of q_len new tokens per sequence: q [B,q_len,h,d_h] bf16.

    K/V bf16, or uint8 E4M3 codes when k_scale and v_scale are given.
    Returns (out [B,q_len,h,d_h] bf16, lse [B,q_len,h] fp32 or None).
    """
    import torch
    B, q_len, h, d_h = q.shape
    h_kv = K.shape[2]
    if block_table is None:
        s_max = K.shape[1] if s_max is None else s_max
        max_blocks, num_blocks = 0, 0
    else:
        max_blocks, num_blocks = block_table.shape[1], K.shape[0]
        s_max = max_blocks * block_size if s_max is None else s_max
    out = torch.empty_like(q)
    l = torch.empty((B, q_len, h), dtype=torch.float32, device=q.device) if lse else None
    ws = workspace or Workspace(q.device)
    wb, wn = ws.get(attn_decode_gqa_multi_workspace_bytes(B, q_len, s_max, h, h_kv, d_h))
    if k_scale is None:
        attn_decode_gqa_multi(out, l, q, K, V, s, block_table, max_blocks, block_size,
                              num_blocks, B, q_len, s_max, h, h_kv, d_h, 2, scale, wb, wn, stream)
    else:
        attn_decode_gqa_multi_fp8(out, l, q, K, V, k_scale, v_scale, s, block_table, max_blocks,
                                  block_size, num_blocks, B, q_len, s_max, h, h_kv, d_h, scale,
                                  wb, wn, stream)
    return out, l
