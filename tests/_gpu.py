"""GPU-test helpers: error metrics, tolerances, sampled oracle references."""
import numpy as np
import torch

import oracle
import synth

# bf16 storage with fp32 accumulation, and fp32 storage
BF16_MAX_ABS, BF16_MEAN_ABS, BF16_REL_RMS = 2e-2, 2e-3, 1e-2
F32_MAX_ABS = 1e-5
LSE_F32 = 1e-5


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def stats(gpu: np.ndarray, ref: np.ndarray):
    d = np.abs(gpu - ref)
    rms_ref = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    rel = np.sqrt(np.mean(d ** 2)) / rms_ref if rms_ref > 0 else 0.0
    return float(d.max(initial=0.0)), float(d.mean()) if d.size else 0.0, float(rel)


def assert_close(gpu: np.ndarray, ref: np.ndarray, b: int, what=""):
    mx, mean, rel = stats(gpu, ref)
    if b == 4:
        assert mx <= F32_MAX_ABS, f"{what}: fp32 max-abs {mx:.3e}"
    else:
        assert mx <= BF16_MAX_ABS, f"{what}: bf16 max-abs {mx:.3e}"
        assert mean <= BF16_MEAN_ABS, f"{what}: bf16 mean-abs {mean:.3e}"
        assert rel <= BF16_REL_RMS, f"{what}: bf16 rel-rms {rel:.3e}"
    return mx, mean, rel


def assert_lse_close(gpu: np.ndarray, ref: np.ndarray, b: int, what=""):
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(gpu)), f"{what}: lse finiteness differs"
    assert np.all(np.isneginf(gpu[~fin])), f"{what}: empty rows must give -inf"
    if fin.any():
        err = np.abs(gpu[fin] - ref[fin])
        mx = float(np.max(err))
        if b == 4:
            assert mx <= LSE_F32 * max(1.0, float(np.max(np.abs(ref[fin])))), f"{what}: lse err {mx:.3e}"
        else:
            # the bf16 bounds on every result: max-abs <= 2e-2, mean-abs <= 2e-3
            # (a sequence of one token has lse = that token's score, which
            # carries the bf16 rounding of the absorbed MLA query unaveraged)
            assert mx <= BF16_MAX_ABS, f"{what}: lse max-abs {mx:.3e}"
            assert float(np.mean(err)) <= BF16_MEAN_ABS, f"{what}: lse mean-abs {np.mean(err):.3e}"


def gqa_sample_reference(d, shape, pairs):
    """Oracle outputs for selected (b, j) KV-head groups of a large input.

    Copies q[b, j*g:(j+1)*g], K/V[b, :s_b, j] (through the block table when
    paged) to the host and runs the oracle on that one-KV-head slice.
    Returns {(b, j): (out [g, d_h], lse [g])}.
    """
    g = shape.h // shape.h_kv
    res = {}
    for (bi, j) in pairs:
        n = int(shape.s[bi])
        q = synth.host_bits(d["q"][bi:bi + 1, j * g:(j + 1) * g])
        if shape.paged:
            tab = d["block_table_host"][bi]
            nb = (n + shape.block_size - 1) // shape.block_size
            idx = torch.as_tensor(tab[:nb], dtype=torch.long, device=d["K"].device)
            Kb = d["K"].index_select(0, idx).reshape(-1, shape.h_kv, shape.d_h)[:max(n, 1), j]
            Vb = d["V"].index_select(0, idx).reshape(-1, shape.h_kv, shape.d_h)[:max(n, 1), j]
        else:
            Kb = d["K"][bi, :max(n, 1), j]
            Vb = d["V"][bi, :max(n, 1), j]
        K = synth.host_bits(Kb)[None, :, None, :]
        V = synth.host_bits(Vb)[None, :, None, :]
        out, lse = oracle.gqa_decode(q, K, V, np.array([n], np.int32), shape.b)
        res[(bi, j)] = (out[0], lse[0])
    return res
