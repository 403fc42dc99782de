"""Shared helpers of the GPU parity tests (comparison bars and row sampling)."""
import numpy as np
import torch

# Output tolerance against the float64 oracle for bf16 attention outputs:
# max |o - ref| <= 1e-2 and sum|o - ref| / sum|ref| <= 2e-3 (mean relative error).
MAX_ABS = 1e-2
MEAN_REL = 2e-3


def gpu_available() -> bool:
    return torch.cuda.is_available()


def out_errors(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got.astype(np.float64) - ref)
    return float(d.max()), float(d.sum() / max(np.abs(ref).sum(), 1e-300))


def assert_out_close(got: np.ndarray, ref: np.ndarray, what=""):
    mx, mr = out_errors(got, ref)
    print(f"  {what}: max_abs={mx:.3e} mean_rel={mr:.3e}", flush=True)
    assert np.isfinite(got).all(), what
    assert mx <= MAX_ABS, f"{what}: max abs {mx}"
    assert mr <= MEAN_REL, f"{what}: mean rel {mr}"


def sample_rows(cu, topk, seed, n_random=32, edge=8):
    """Rows that cover each sequence's start, the last rows with fewer than k keys, the first
    rows with more, its end, frame boundaries of 1024-token frames, and seeded random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(len(cu) - 1):
        a, e = int(cu[b]), int(cu[b + 1])
        L = e - a
        if L == 0:
            continue
        for i in list(range(min(edge, L))) + list(range(max(0, L - edge), L)):
            rows.add(a + i)
        for i in range(max(0, topk - edge), min(L, topk + edge)):
            rows.add(a + i)
        for f in range(1024, L, 1024 * 17):
            rows.update({a + f - 1, a + f, a + f + 16})
        rows.update((a + rng.integers(0, L, size=max(1, n_random // (len(cu) - 1)))).tolist())
    return np.array(sorted(r for r in rows if r < int(cu[-1])), dtype=np.int64)


def survey_sample_rows(cu, seed, edge=2048, n_random=4096, frame=1024, text=16):
    """The deterministic row sample of the long workloads: each sequence's first and last
    ``edge`` rows; at every frame boundary the last row of the previous frame, the frame's first
    (timestamp-text) row and its first vision row; and ``n_random`` seeded rows over the batch."""
    rng = np.random.default_rng(seed)
    rows = set()
    T = int(cu[-1])
    for b in range(len(cu) - 1):
        a, e = int(cu[b]), int(cu[b + 1])
        L = e - a
        rows.update(range(a, a + min(edge, L)))
        rows.update(range(max(a, e - edge), e))
        for f in range(frame, L, frame):
            rows.update(a + r for r in (f - 1, f, f + text) if r < L)
    if n_random and T:
        rows.update(rng.integers(0, T, size=n_random).tolist())
    return np.array(sorted(rows), dtype=np.int64)
