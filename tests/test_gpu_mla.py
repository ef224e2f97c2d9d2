"""GPU parity of attn_decode_mla_absorbed against the CPU oracle (absorbed
form, itself pinned to explicit K/V expansion).  Output and u_latent use the
bf16 tolerances (max-abs <= 2e-2, mean-abs <= 2e-3, rel-RMS <= 1e-2); the
kernel rounds the absorbed query and the probabilities to bf16 for the
matrix cores and accumulates in fp32."""
import numpy as np
import pytest
import torch

import decode_attention_kv_attn_amd as A
import oracle
import synth
from tests._gpu import assert_close, assert_lse_close, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(sh, sample=None):
    print(f"[mla] {sh.name} B={sh.B} h={sh.h} s={list(sh.s)[:6]} paged={sh.paged}", flush=True)
    d = synth.draw_mla(sh, device=DEV)
    out, ul, lse = A.decode_mla(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["cache"], d["s"],
                                block_table=d.get("block_table"), s_max=sh.s_max)
    torch.cuda.synchronize()
    bs = range(sh.B) if sample is None else sample
    for bi in bs:
        n = int(sh.s[bi])
        args = [synth.host_bits(d[k][bi:bi + 1]) for k in ("q_nope", "q_rope")]
        w = [synth.host_bits(d["w_uk"]), synth.host_bits(d["w_uv"])]
        if sh.paged:
            tab = d["block_table_host"][bi]
            nb = (n + sh.block_size - 1) // sh.block_size
            idx = torch.as_tensor(tab[:nb], dtype=torch.long, device=DEV)
            rows = d["cache"].index_select(0, idx).reshape(-1, sh.d_c + sh.d_R)[:max(n, 1)]
        else:
            rows = d["cache"][bi, :max(n, 1)]
        C = synth.host_bits(rows)[None]
        ro, ru, rl = oracle.mla_absorbed(args[0], args[1], w[0], w[1], C,
                                         np.array([n], np.int32))
        assert_close(to_f64(out[bi:bi + 1]), ro, 2, f"out b={bi}")
        assert_close(to_f64(ul[bi:bi + 1]), ru, 2, f"u_latent b={bi}")
        assert_lse_close(to_f64(lse[bi:bi + 1]), rl, 2, f"lse b={bi}")
    return d, out, ul, lse


def shape(B, h, s, paged=False, seed=31, d_nope=128, d_v=128):
    return synth.MlaShape("t", B=B, h=h, d_c=512, d_R=64, d_nope=d_nope, d_v=d_v, s=tuple(s),
                          paged=paged, seed=seed)


@pytest.mark.parametrize("h", [16, 32, 48, 128])
def test_head_counts(h):
    run(shape(2, h, (77, 300), seed=h))


@pytest.mark.parametrize("s", [(1, 2), (31, 33), (0, 64), (0, 0), (1000, 17)])
def test_lengths_ragged_empty(s):
    run(shape(2, 32, s, seed=sum(s) + 1))


def test_batch_not_multiple_of_16_and_other_dims():
    run(shape(19, 16, tuple(range(5, 5 + 19 * 7, 7)), seed=5, d_nope=64, d_v=32))


def test_long_context_split():
    run(shape(1, 128, (12000,), seed=6))


def test_many_partials_per_sequence():
    # ~240 workgroups share one sequence: the merge folds its partials in
    # several chunks on each of the wavefronts that split them
    run(shape(1, 16, (70000,), seed=43))


def test_nine_sequences_wide_value():
    # one full block of 8 sequences and one of a single sequence; d_v = 256
    # gives each wavefront two output column tiles
    run(shape(9, 16, tuple(range(300, 300 + 9 * 450, 450)), seed=44, d_v=256))


# The decode tile schedule gives each of the 256 workgroups an equal run of
# 32-token tiles across sequence boundaries (at least 8 tiles).  Many short
# sequences put several sequences, empty ones among them, into one
# workgroup; uneven long ones split a sequence over several workgroups.
def test_schedule_many_short_sequences_per_workgroup():
    rng = np.random.default_rng(40)
    s = tuple(int(x) for x in rng.integers(0, 70, size=300))
    run(shape(300, 16, s, seed=40), sample=list(range(0, 300, 7)) + [299])


def test_schedule_uneven_lengths():
    run(shape(6, 32, (1, 9000, 33, 0, 2048, 31), seed=41))


def test_schedule_paged_mixed():
    rng = np.random.default_rng(42)
    s = tuple(int(x) for x in rng.integers(0, 3000, size=40))
    run(shape(40, 32, s, paged=True, seed=42), sample=[0, 7, 13, 21, 39])


def test_paged_shuffled():
    run(shape(4, 32, (1, 16, 17, 700), paged=True, seed=7))


def test_paged_bit_identical_to_identity_table():
    s = (5, 40, 129, 700)
    sh = shape(4, 64, s, paged=True, seed=8)
    d = synth.draw_mla(sh, device=DEV)
    tab = d["block_table_host"]
    ident, _ = synth.identity_table(s, 16)
    order = torch.as_tensor(np.concatenate([tab[i, :(n + 15) // 16] for i, n in enumerate(s)]),
                            dtype=torch.long, device=DEV)
    Ci = d["cache"].index_select(0, order)
    a = A.decode_mla(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["cache"], d["s"],
                     block_table=d["block_table"], s_max=max(s))
    b = A.decode_mla(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], Ci, d["s"],
                     block_table=torch.from_numpy(ident).to(DEV), s_max=max(s))
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


def test_deepseek_v3_full_size_sampled():
    sh = synth.configs()["deepseek_v3_mla"]
    run(sh, sample=[0, 17, sh.B - 1])


def test_paged_mla_full_size_sampled():
    sh = synth.configs()["paged_mla"]
    lens = np.asarray(sh.s)
    pick = [int(np.argmin(lens)), int(np.argmax(lens)), 64]
    run(sh, sample=pick)


def test_peaked_logits_take_the_rescaling_path():
    # Tokens whose latent row points along head 0's absorbed query: each
    # logit exceeds its tile run's first maximum by far more than 2^64 in
    # probability ratio, so the workgroup holding it stops and its partials
    # are recomputed with online rescaling.  With 167 tiles over 256
    # workgroups every workgroup takes 8 tiles: token 200 sits in the middle
    # of workgroup 0's run, token 80 of sequence 1 in the middle of
    # workgroup 1's run after it has finished sequence 0's last two tiles,
    # and token 4000 on the last tile of workgroup 16's run.
    sh = shape(2, 128, (300, 5000), seed=71)
    d = synth.draw_mla(sh, device=DEV)
    qt = torch.matmul(d["q_nope"][:, 0].float(), d["w_uk"][0].float())   # q~ of head 0
    for bi, t in ((0, 200), (1, 80), (1, 4000)):
        c = qt[bi] / qt[bi].norm() * 40.0
        r = d["q_rope"][bi, 0].float()
        kr = r / r.norm() * 40.0
        d["cache"][bi, t] = torch.cat([c, kr]).to(torch.bfloat16)
    out, ul, lse = A.decode_mla(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["cache"], d["s"])
    torch.cuda.synchronize()
    for bi in range(2):
        n = int(sh.s[bi])
        args = [synth.host_bits(d[k][bi:bi + 1]) for k in ("q_nope", "q_rope")]
        ro, ru, rl = oracle.mla_absorbed(args[0], args[1], synth.host_bits(d["w_uk"]),
                                         synth.host_bits(d["w_uv"]),
                                         synth.host_bits(d["cache"][bi, :n])[None],
                                         np.array([n], np.int32))
        assert rl[0, 0] > 50            # the spike dominates head 0
        assert_close(to_f64(out[bi:bi + 1]), ro, 2, f"out b={bi}")
        assert_close(to_f64(ul[bi:bi + 1]), ru, 2, f"u_latent b={bi}")
        assert_lse_close(to_f64(lse[bi:bi + 1]), rl, 2, f"lse b={bi}")


def test_large_batch_short_sequences():
    rng = np.random.default_rng(45)
    s = tuple(int(x) for x in rng.integers(0, 120, size=1200))
    run(shape(1200, 16, s, seed=45), sample=[0, 1, 599, 1199])


def _align256(x):
    return (x + 255) // 256 * 256


def _expected_schedule(seen, n_wg=256, min_tiles=8, kT=32):
    """The equal-tile schedule from its rule: the tiles of all query rows end
    to end, tile_start = exclusive prefix sums, tpw = max(ceil(total / n_wg),
    min_tiles), and workgroup w starts in the row holding tile w * tpw (-1
    once past the total)."""
    tiles = [(n + kT - 1) // kT for n in seen]
    ts = np.concatenate([[0], np.cumsum(tiles)]).astype(np.int64)
    total = int(ts[-1])
    tpw = max(-(-total // n_wg), min_tiles)
    wstart = []
    for w in range(n_wg):
        t = w * tpw
        if t >= total:
            wstart.append(-1)
        else:
            wstart.append(int(np.searchsorted(ts, t, side="right") - 1))
    return np.concatenate([ts, wstart, [tpw]]).astype(np.int32)


@pytest.mark.parametrize("B,q_len,hi", [(32, 1, 8192), (1100, 1, 300), (7, 3, 2000), (1, 1, 0)])
def test_schedule_metadata_bit_exact(B, q_len, hi):
    # the tile schedule the absorb launch writes into the workspace, against
    # the rule it implements (more than 1,024 rows take several chunks of
    # the one workgroup that computes it; several new tokens per sequence
    # count the tokens each position sees)
    rng = np.random.default_rng(44 + B)
    s = [int(x) for x in rng.integers(0, hi + 1, size=B)]
    if B > 3:
        s[1], s[2] = 0, 1
    h, d_c, d_R = 16, 512, 64
    sh = synth.MlaShape("t", B=B, h=h, d_c=d_c, d_R=d_R, d_nope=128, d_v=128, s=tuple(s),
                        seed=44, q_len=q_len)
    print(f"[mla-schedule] B={B} q_len={q_len}", flush=True)
    d = synth.draw_mla(sh, device=DEV)
    ws = A.Workspace(DEV)
    if q_len == 1:
        A.decode_mla(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["cache"], d["s"],
                     s_max=sh.s_max, workspace=ws)
    else:
        A.decode_mla_multi(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["cache"], d["s"],
                           s_max=sh.s_max, workspace=ws)
    torch.cuda.synchronize()
    rows, n_wg = B * q_len, 256
    slots = n_wg + rows - 1
    off = (65536 + _align256(rows * ((h + 31) // 32) * 32 * (d_c + d_R) * 2)
           + _align256(slots * h * d_c * 2) + _align256(slots * h * 2 * 4) + _align256(n_wg * 4))
    n = rows + 1 + n_wg + 1
    got = ws.buf[off:off + 4 * n].cpu().numpy().view(np.int32)
    seen = [max(min(s[r // q_len], sh.s_max) - (q_len - 1 - r % q_len), 0) for r in range(rows)]
    want = _expected_schedule(seen)
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:10]
