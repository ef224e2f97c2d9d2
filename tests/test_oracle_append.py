"""Pins for the append oracle: the new row lands at slot pos_b (contiguous)
or at block_table[b][pos_b / 16] * 16 + pos_b % 16 (paged), nothing else
changes.  Appending by concatenation is the decode step of the absorbed
module on the llms.blog MLA page; the paged placement follows "What a paged
KV cache block holds" (charlestar.github.io)."""
import numpy as np

import oracle
import synth
from tests._util import stored


def test_contiguous_append_places_rows():
    rng = np.random.default_rng(1)
    B, s_max, h_kv, d = 3, 10, 2, 8
    K = stored(rng.standard_normal((B, s_max, h_kv, d)), 2)
    V = stored(rng.standard_normal((B, s_max, h_kv, d)), 2)
    kn = stored(rng.standard_normal((B, h_kv, d)), 2)
    vn = stored(rng.standard_normal((B, h_kv, d)), 2)
    pos = np.array([0, 9, 4], dtype=np.int32)
    K2, V2 = oracle.kv_append(K, V, kn, vn, pos, 2)
    for bi in range(B):
        assert np.array_equal(K2[bi, pos[bi]], kn[bi])
        assert np.array_equal(V2[bi, pos[bi]], vn[bi])
    mask = np.ones((B, s_max), bool)
    mask[np.arange(B), pos] = False
    assert np.array_equal(K2[mask], K[mask]) and np.array_equal(V2[mask], V[mask])


def test_paged_append_follows_table_and_mla_has_no_v():
    rng = np.random.default_rng(2)
    s = (5, 16, 31)
    tab, n_blk = synth.block_table(tuple(x + 1 for x in s), 16, seed=3)
    W = 576
    pool = stored(rng.standard_normal((n_blk, 16, 1, W)), 2)
    new = stored(rng.standard_normal((3, 1, W)), 2)
    pos = np.array(s, dtype=np.int32)
    P2, none = oracle.kv_append(pool, None, new, None, pos, 2, block_table=tab)
    assert none is None
    touched = set()
    for bi, p in enumerate(pos):
        blk, off = tab[bi, p // 16], p % 16
        assert np.array_equal(P2[blk, off], new[bi])
        touched.add((blk, off))
    for blk in range(n_blk):
        for off in range(16):
            if (blk, off) not in touched:
                assert np.array_equal(P2[blk, off], pool[blk, off])
