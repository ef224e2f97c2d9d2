"""CPU-side checks of the C ABI: the library loads, exports every entry
point the headers in include/ declare, and its host-only helpers and argument
checks behave (no kernel is launched here)."""
import ctypes as C
import json
import os
import re

import pytest

import decode_attention_kv_attn_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "cell_sizes.json")))


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:size_t|int|const char\*)\s+(\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_header_declares_the_three_entry_points_and_helpers():
    names = declared_functions()
    for n in ("attn_decode_gqa", "attn_decode_mla_absorbed", "kv_cache_append",
              "attn_decode_workspace_bytes", "attn_kv_cell_bytes", "attn_mla_cell_bytes",
              "attn_last_error"):
        assert n in names
    assert sorted(A.EXPORTED) == names


def test_library_exports_every_declared_symbol():
    lib = A.lib()
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = os.popen(f"nm -D --defined-only {A.LIB_PATH}").read()
    for n in declared_functions():
        assert re.search(rf"\bT {n}\b", out), n


def test_library_is_built_for_gfx950():
    blob = open(A.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


@pytest.mark.parametrize("case", GOLD["gqa"], ids=lambda c: c["name"])
def test_kv_cell_bytes_matches_printed(case):
    assert A.attn_kv_cell_bytes(case["L"], case["h_kv"], case["d_h"], case["b"]) * case["tokens"] \
        == case["bytes"]


@pytest.mark.parametrize("case", GOLD["mla"], ids=lambda c: c["name"])
def test_mla_cell_bytes_matches_printed(case):
    assert A.attn_mla_cell_bytes(case["L"], case["d_c"], case["d_R"], case["b"]) * case["tokens"] \
        == case["bytes"]


def test_cell_helpers_reject_negative():
    assert A.attn_kv_cell_bytes(-1, 8, 128, 2) == 0
    assert A.attn_mla_cell_bytes(61, -512, 64, 2) == 0


def test_workspace_bytes():
    # a batch big enough to fill the GPU needs no split, hence no workspace
    assert A.attn_decode_workspace_bytes(0, 4096, 4096, 8, 8, 128) == 0
    # long context, small batch: split-KV partials
    ws = A.attn_decode_workspace_bytes(0, 1, 131072, 64, 8, 128)
    assert ws >= 64 * 2 * 130 * 4
    assert A.attn_decode_workspace_bytes(0, 1, 131072, 64, 7, 128) == 0   # h % h_kv != 0
    mla = A.attn_decode_workspace_bytes(1, 32, 8192, 128, 1, 512, 64)
    assert mla >= 32 * 128 * 576 * 2 + 32 * 128 * 512 * 4


FAKE = 256  # never dereferenced: every call below is rejected before any launch


def gqa_call(**kw):
    args = dict(out=FAKE, lse=None, q=FAKE, cache_k=FAKE, cache_v=FAKE, s=FAKE, block_table=None,
                max_blocks=0, block_size=16, num_blocks=0, B=2, s_max=64, h=8, h_kv=2, d_h=128,
                b=2, scale=0.0, workspace=None, workspace_bytes=0, stream=0, check=False)
    args.update(kw)
    return A.attn_decode_gqa(**args)


def test_gqa_argument_errors():
    assert gqa_call(out=None) == A.ATTN_EINVAL
    assert gqa_call(h=6, h_kv=4) == A.ATTN_EINVAL
    assert "not divisible" in A.attn_last_error()
    assert gqa_call(b=3) == A.ATTN_EINVAL
    assert gqa_call(d_h=96) == A.ATTN_ENOTSUP
    assert gqa_call(b=4, d_h=128) == A.ATTN_ENOTSUP
    assert gqa_call(block_table=FAKE, block_size=24, max_blocks=4, num_blocks=8) == A.ATTN_EINVAL
    assert gqa_call(block_table=FAKE, block_size=16, max_blocks=2, num_blocks=8) == A.ATTN_EINVAL
    # long context at B=1 needs a workspace
    assert gqa_call(B=1, s_max=65536) == A.ATTN_EWORKSPACE
    assert "workspace" in A.attn_last_error()


def mla_call(**kw):
    args = dict(out=FAKE, u_latent=None, lse=None, q_nope=FAKE, q_rope=FAKE, w_uk=FAKE, w_uv=FAKE,
                cache=FAKE, s=FAKE, block_table=None, max_blocks=0, block_size=16, num_blocks=0,
                B=2, s_max=64, h=128, d_c=512, d_R=64, d_nope=128, d_v=128, b=2, scale=0.0,
                workspace=None, workspace_bytes=0, stream=0, check=False)
    args.update(kw)
    return A.attn_decode_mla_absorbed(**args)


def test_mla_argument_errors():
    assert mla_call(cache=None) == A.ATTN_EINVAL
    assert mla_call(b=4) == A.ATTN_ENOTSUP
    assert mla_call(d_c=256) == A.ATTN_ENOTSUP
    assert mla_call(h=24) == A.ATTN_ENOTSUP
    assert mla_call() == A.ATTN_EWORKSPACE


def test_append_argument_errors():
    kw = dict(cache_k=FAKE, cache_v=FAKE, k_new=FAKE, v_new=None, pos=FAKE, block_table=None,
              max_blocks=0, block_size=16, num_blocks=0, B=2, s_max=8, h_kv=2, d_h=64, b=2,
              stream=0, check=False)
    assert A.kv_cache_append(**kw) == A.ATTN_EINVAL          # v_new missing
    kw.update(v_new=FAKE, b=8)
    assert A.kv_cache_append(**kw) == A.ATTN_EINVAL
    kw.update(b=2, s_max=0)
    assert A.kv_cache_append(**kw) == A.ATTN_EINVAL


def test_stream_probe_rejects_bad_arguments():
    unit = 2048 * 16384
    assert A.attn_stream_read_probe(None, unit, FAKE, stream=0, check=False) == A.ATTN_EINVAL
    assert A.attn_stream_read_probe(FAKE, unit, None, stream=0, check=False) == A.ATTN_EINVAL
    assert A.attn_stream_read_probe(FAKE, 0, FAKE, stream=0, check=False) == A.ATTN_EINVAL
    assert A.attn_stream_read_probe(FAKE, unit + 16, FAKE, stream=0, check=False) == A.ATTN_EINVAL
    assert "multiple" in A.attn_last_error()


def test_fp8_gqa_argument_errors():
    kw = dict(out=FAKE, lse=None, q=FAKE, cache_k=FAKE, cache_v=FAKE, k_scale=0.5, v_scale=0.5,
              s=FAKE, block_table=None, max_blocks=0, block_size=16, num_blocks=0, B=2, s_max=64,
              h=8, h_kv=2, d_h=128, scale=0.0, workspace=None, workspace_bytes=0, stream=0,
              check=False)
    for bad in (dict(k_scale=0.0), dict(v_scale=-1.0), dict(k_scale=float("inf")),
                dict(v_scale=float("nan"))):
        assert A.attn_decode_gqa_fp8(**{**kw, **bad}) == A.ATTN_EINVAL, bad
    assert A.attn_decode_gqa_fp8(**{**kw, "h": 128, "h_kv": 1}) == A.ATTN_ENOTSUP   # g > 64
    assert A.attn_decode_gqa_fp8(**{**kw, "d_h": 96}) == A.ATTN_ENOTSUP
    assert A.attn_decode_gqa_fp8(**{**kw, "B": 1, "s_max": 65536}) == A.ATTN_EWORKSPACE


def multi_call(**kw):
    args = dict(out=FAKE, lse=None, q=FAKE, cache_k=FAKE, cache_v=FAKE, s=FAKE, block_table=None,
                max_blocks=0, block_size=16, num_blocks=0, B=2, q_len=4, s_max=64, h=8, h_kv=2,
                d_h=128, b=2, scale=0.0, workspace=None, workspace_bytes=0, stream=0, check=False)
    args.update(kw)
    return A.attn_decode_gqa_multi(**args)


def test_multi_token_argument_errors_and_workspace():
    assert multi_call(q_len=0) == A.ATTN_EINVAL
    assert multi_call(q_len=65) == A.ATTN_EINVAL
    assert multi_call(b=4) == A.ATTN_ENOTSUP
    assert multi_call(b=1) == A.ATTN_ENOTSUP          # FP8 has its own entry point
    assert multi_call(h=6, h_kv=4) == A.ATTN_EINVAL
    assert multi_call(B=1, s_max=65536) == A.ATTN_EWORKSPACE
    # partials for every (position, head) row of every split
    ws1 = A.attn_decode_gqa_multi_workspace_bytes(1, 1, 65536, 64, 8, 128)
    ws4 = A.attn_decode_gqa_multi_workspace_bytes(1, 4, 65536, 64, 8, 128)
    assert ws1 > 0 and ws4 >= 4 * 64 * 2 * (128 + 2) * 4
    assert A.attn_decode_gqa_multi_workspace_bytes(1, 0, 64, 8, 2, 128) == 0
    assert A.attn_decode_gqa_multi_workspace_bytes(1, 65, 64, 8, 2, 128) == 0
    assert A.attn_decode_gqa_multi_workspace_bytes(1, 2, 64, 6, 4, 128) == 0
    # for q_len = 1 the plan is the single-token one, whose workspace query covers it
    assert ws1 <= A.attn_decode_workspace_bytes(0, 1, 65536, 64, 8, 128)


def test_merge_argument_errors():
    kw = dict(out=FAKE, lse=None, o_parts=FAKE, lse_parts=FAKE, n_parts=4, B=2, h=8, d=128,
              b_parts=2, b_out=2, stream=0, check=False)
    assert A.attn_merge_partials(**{**kw, "out": None}) == A.ATTN_EINVAL
    assert A.attn_merge_partials(**{**kw, "n_parts": 0}) == A.ATTN_EINVAL
    assert A.attn_merge_partials(**{**kw, "h": 0}) == A.ATTN_EINVAL
    assert A.attn_merge_partials(**{**kw, "d": 6}) == A.ATTN_ENOTSUP
    assert A.attn_merge_partials(**{**kw, "d": 2048}) == A.ATTN_ENOTSUP
    assert A.attn_merge_partials(**{**kw, "b_parts": 1}) == A.ATTN_ENOTSUP
    assert A.attn_merge_partials(**{**kw, "o_parts": FAKE + 8}) == A.ATTN_EINVAL   # not 16-byte aligned
    assert A.attn_merge_partials(**{**kw, "B": 0}) == A.ATTN_OK                   # nothing to merge


def test_mla_fp8_and_fp8_append_argument_errors():
    kw = dict(out=FAKE, u_latent=None, lse=None, q_nope=FAKE, q_rope=FAKE, w_uk=FAKE, w_uv=FAKE,
              cache=FAKE, c_scale=0.5, r_scale=0.5, s=FAKE, block_table=None, max_blocks=0,
              block_size=16, num_blocks=0, B=2, s_max=64, h=128, d_c=512, d_R=64, d_nope=128,
              d_v=128, scale=0.0, workspace=None, workspace_bytes=0, stream=0, check=False)
    assert A.attn_decode_mla_absorbed_fp8(**{**kw, "c_scale": 0.0}) == A.ATTN_EINVAL
    assert A.attn_decode_mla_absorbed_fp8(**{**kw, "r_scale": float("inf")}) == A.ATTN_EINVAL
    assert A.attn_decode_mla_absorbed_fp8(**{**kw, "d_c": 256}) == A.ATTN_ENOTSUP
    assert A.attn_decode_mla_absorbed_fp8(**kw) == A.ATTN_EWORKSPACE
    ak = dict(cache=FAKE, kv_new=FAKE, c_scale=0.5, r_scale=0.5, pos=FAKE, block_table=None,
              max_blocks=0, block_size=16, num_blocks=0, B=2, s_max=8, d_c=512, d_R=64, stream=0,
              check=False)
    assert A.kv_cache_append_mla_fp8(**{**ak, "r_scale": 0.0}) == A.ATTN_EINVAL
    assert A.kv_cache_append_mla_fp8(**{**ak, "d_c": 510}) == A.ATTN_EINVAL
    assert A.kv_cache_append_mla_fp8(**{**ak, "kv_new": None}) == A.ATTN_EINVAL
    fk = dict(cache_k=FAKE, cache_v=FAKE, k_new=FAKE, v_new=FAKE, k_scale=0.5, v_scale=0.5,
              pos=FAKE, block_table=None, max_blocks=0, block_size=16, num_blocks=0, B=2, s_max=8,
              h_kv=2, d_h=64, stream=0, check=False)
    assert A.kv_cache_append_fp8(**{**fk, "v_scale": -2.0}) == A.ATTN_EINVAL
    assert A.kv_cache_append_fp8(**{**fk, "v_new": None}) == A.ATTN_EINVAL


def test_mla_multi_and_output_path_argument_errors_and_workspace():
    mk = dict(out=FAKE, u_latent=None, lse=None, q_nope=FAKE, q_rope=FAKE, w_uk=FAKE, w_uv=FAKE,
              cache=FAKE, s=FAKE, block_table=None, max_blocks=0, block_size=16, num_blocks=0,
              B=2, q_len=2, s_max=64, h=128, d_c=512, d_R=64, d_nope=128, d_v=128, b=2,
              scale=0.0, workspace=None, workspace_bytes=0, stream=0, check=False)
    assert A.attn_decode_mla_absorbed_multi(**{**mk, "q_len": 0}) == A.ATTN_EINVAL
    assert A.attn_decode_mla_absorbed_multi(**{**mk, "q_len": 1025}) == A.ATTN_EINVAL
    assert A.attn_decode_mla_absorbed_multi(**mk) == A.ATTN_EWORKSPACE
    # q_len = 1 needs exactly the single-token workspace
    assert (A.attn_decode_mla_multi_workspace_bytes(4, 1, 128, 512, 64)
            == A.attn_decode_workspace_bytes(1, 4, 64, 128, 1, 512, 64))
    assert (A.attn_decode_mla_multi_workspace_bytes(4, 3, 128, 512, 64)
            == A.attn_decode_workspace_bytes(1, 12, 64, 128, 1, 512, 64))
    ok = dict(out=FAKE, lse=None, q_nope=FAKE, q_rope=FAKE, w_uk=FAKE, w_uv=FAKE, w_o=FAKE,
              cache=FAKE, s=FAKE, block_table=None, max_blocks=0, block_size=16, num_blocks=0,
              B=2, q_len=1, s_max=64, h=128, d_c=512, d_R=64, d_nope=128, d_v=128, d_model=5120,
              b=2, scale=0.0, workspace=None, workspace_bytes=0, stream=0, check=False)
    assert A.attn_decode_mla_out(**{**ok, "d_model": 100}) == A.ATTN_ENOTSUP
    assert A.attn_decode_mla_out(**{**ok, "w_o": None}) == A.ATTN_EINVAL
    assert A.attn_decode_mla_out(**{**ok, "b": 4}) == A.ATTN_ENOTSUP
    assert A.attn_decode_mla_out(**ok) == A.ATTN_EWORKSPACE
    assert A.attn_decode_mla_out(**{**ok, "B": 0}) == A.ATTN_OK
    wd = A.attn_decode_mla_out_workspace_bytes(0, 32, 1, 128, 512, 64, 128, 5120)
    wm = A.attn_decode_mla_out_workspace_bytes(1, 32, 1, 128, 512, 64, 0, 5120)
    base = A.attn_decode_workspace_bytes(1, 32, 64, 128, 1, 512, 64)
    assert wd >= base + 32 * 128 * 128 * 2 and wm >= base + 32 * 128 * 512 * 2
    assert A.attn_decode_mla_out_workspace_bytes(0, 32, 1, 128, 512, 64, 128, 100) == 0
    pm = dict(w_absorbed=FAKE, w_o=FAKE, w_uv=FAKE, h=128, d_c=512, d_v=128, d_model=5120,
              stream=0, check=False)
    assert A.attn_mla_premerge_weights(**{**pm, "w_uv": None}) == A.ATTN_EINVAL
    assert A.attn_mla_premerge_weights(**{**pm, "d_c": 320}) == A.ATTN_ENOTSUP
    assert A.attn_mla_premerge_weights(**{**pm, "d_v": 512}) == A.ATTN_ENOTSUP


def test_output_form_choice():
    # DeepSeek shapes: the merged weight is d_c / d_v = 4 times W_O, so the
    # deferred form moves less at every batch size
    for B in (1, 32, 1024):
        assert A.attn_mla_out_form(B, 1, 128, 512, 128, 5120) == 0
    # a latent narrower than the value heads: the merged weight is the smaller one
    assert A.attn_mla_out_form(32, 1, 8, 64, 128, 4096) == 1
    assert A.attn_mla_out_form(0, 1, 8, 64, 128, 4096) == -1


def test_mla_mode_choice():
    # measured crossovers: absorbed for decode-sized query blocks, MHA mode
    # for prefill-sized ones, later for longer contexts
    assert A.attn_mla_mode(1, 8192) == 0 and A.attn_mla_mode(64, 2048) == 0
    assert A.attn_mla_mode(256, 2048) == 1 and A.attn_mla_mode(256, 8192) == 0
    assert A.attn_mla_mode(1024, 8192) == 1
    assert A.attn_mla_mode(0, 8192) == -1
    # the 64 KiB arrival-counter prefix every workspace keeps, then K and V
    assert A.attn_decode_mla_mha_workspace_bytes(4, 8192, 128) == 65536 + 2 * 4 * 8192 * 128 * 128 * 2
