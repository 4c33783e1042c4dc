"""Helpers for the GPU-vs-oracle parity tests (imported by tests only)."""
from __future__ import annotations

import numpy as np
import torch

# Tolerance for bf16 inputs with fp32 accumulation, over the compared output
# elements: max-abs and mean-abs error against the fp64 oracle.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
# lse = m + ln(d).  The kernels accumulate d from the same bf16-rounded
# weights that multiply V: bf16 keeps 8 significant bits, so round-to-nearest
# changes each weight by a relative <= 2^-8 (the unit roundoff) and a sum of
# such weights by a relative <= 2^-8 too; with fp32 logits and fp32
# accumulation around it, |dlse| <= ln(1 + 2^-8) ~ 3.9e-3.
LSE_ABS = 4e-3


def assert_close(gpu: torch.Tensor | np.ndarray, ref: np.ndarray, *, what: str,
                 max_abs: float = MAX_ABS, mean_abs: float = MEAN_ABS):
    g = gpu.detach().double().cpu().numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    g = g.reshape(ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values in the GPU output"
    err = np.abs(g - ref)
    mx, mn = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    assert mx <= max_abs and mn <= mean_abs, \
        f"{what}: max-abs {mx:.3e} (bound {max_abs:g}), mean-abs {mn:.3e} (bound {mean_abs:g})"
    return mx, mn


def assert_lse_close(gpu: torch.Tensor, ref: np.ndarray, *, what: str, atol: float = LSE_ABS):
    g = gpu.detach().double().cpu().numpy().reshape(ref.shape)
    inf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(g), inf_ref), f"{what}: -inf pattern differs"
    fin = ~inf_ref
    err = np.abs(g[fin] - ref[fin])
    assert np.all(np.isfinite(g[fin])) and (err.size == 0 or err.max() <= atol), \
        f"{what}: lse max-abs {err.max() if err.size else 0:.3e} > {atol:g}"


def sample_prefill_rows(cu_seqlens, num_q_heads: int, n_random: int, seed: int,
                        all_heads_positions: int = 2):
    """(token, head) pairs: every sequence's tile-boundary and tail rows, a few
    positions with every head, and random rows; each head appears at least once."""
    rng = np.random.default_rng(seed)
    cu = [int(x) for x in cu_seqlens]
    rows = set()
    for s in range(len(cu) - 1):
        a, n = cu[s], cu[s + 1] - cu[s]
        if n == 0:
            continue
        picks = {0, 1, 31, 32, 33, 63, 64, 65, 127, 128, n - 1, n - 2, n - 32, n - 33, n // 2}
        for p in picks:
            if 0 <= p < n:
                rows.add((a + p, int(rng.integers(num_q_heads))))
        for p in rng.integers(0, n, size=all_heads_positions):
            for h in range(num_q_heads):
                rows.add((a + int(p), h))
    T = cu[-1]
    for _ in range(n_random):
        rows.add((int(rng.integers(T)), int(rng.integers(num_q_heads))))
    for h in range(num_q_heads):
        rows.add((int(rng.integers(T)), h))
    return sorted(rows)


def gather_rows(out: torch.Tensor, rows) -> torch.Tensor:
    """out [T, Hq, D] (GPU) -> [n, D] on the CPU for the given (token, head) rows."""
    idx = torch.tensor(rows, dtype=torch.long)
    return out.detach().cpu()[idx[:, 0], idx[:, 1]]
