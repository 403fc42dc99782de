"""GPU parity of the standalone top-k (dsa_topk, through the C ABI) against its CPU oracle.

Bar: the selected positions are bit-exact (integer output).  Cases cover special values
(NaN of any sign and payload, +-inf, +-0), every path of the kernel (all selectable kept;
candidates finished in LDS; a second-digit refinement when the threshold digit is crowded;
the HBM fallback for massive ties), ragged row lengths, rows shorter than k, empty rows,
unaligned rows, and the full-size workload on sampled rows.  Rows of 8192 keys or more take a
sampled single pass first (falling back to the two-pass path on any miss); the long cases
cover it with special values and with more than k ties at +inf."""
import zlib

import numpy as np
import pytest
import torch

from oracle.topk_general import topk_general
from sparse_attention_long_04_amd import dsa, workloads
from sparse_attention_long_04_amd import inputs as gen

from gpu_util import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _run(scores: np.ndarray, k: int, lens=None, ld=None, offset=0):
    rows, n = scores.shape
    ld = n if ld is None else ld
    buf = np.full(offset + rows * ld + 4, np.float32(7.0), dtype=np.float32)
    for r in range(rows):
        buf[offset + r * ld: offset + r * ld + n] = scores[r]
    dev = torch.from_numpy(buf).cuda()
    out = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    ln = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    dsa.dsa_topk(dev.data_ptr() + 4 * offset, rows, n, ld, ln, k, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = [
    # name, rows, n, kind, special fractions, ks
    ("normal", 8, 5000, "normal", dict(), (1, 100, 2048, 5000, 6000)),
    ("specials", 16, 3000, "ties", dict(masked=0.1, nans=0.1, infs=0.02, zeros=0.1), (1, 7, 256, 2048)),
    ("narrow_refine", 4, 40000, "narrow", dict(), (2048,)),
    ("narrow_refine_masked", 4, 40000, "narrow", dict(masked=0.3, nans=0.05), (100, 2048)),
    ("ties_hbm_fallback", 4, 30000, "ties", dict(), (1, 2048, 4096)),
    ("const", 3, 20000, "const", dict(), (2048,)),
    ("all_masked", 2, 1000, "normal", dict(masked=0.6, nans=0.5), (16, 2048)),
    ("long_normal", 4, 131072, "normal", dict(masked=0.01), (2048,)),
    # rows of 8192+ keys take the sampled single pass first
    ("long_specials", 4, 50000, "normal", dict(masked=0.1, nans=0.1, infs=0.01, zeros=0.2), (1, 64, 2048)),
    ("long_posinf_ties", 3, 40000, "normal", dict(infs=0.2), (2048,)),  # k among > k ties at +inf
]


@pytest.mark.parametrize("name,rows,n,kind,sp,ks", CASES, ids=[c[0] for c in CASES])
def test_topk_general_parity(name, rows, n, kind, sp, ks):
    s = gen.make_topk_scores(rows, n, seed=zlib.crc32(name.encode()) % 1000, kind=kind, **sp)
    for k in ks:
        print(f"[topk] {name} rows={rows} n={n} k={k}", flush=True)
        got = _run(s, k)
        ref = topk_general(s, k)
        bad = [r for r in range(rows) if not np.array_equal(got[r], ref[r])]
        assert not bad, f"{name} k={k}: rows {bad}"


def test_topk_general_ragged_lengths_and_stride():
    s = gen.make_topk_scores(9, 9000, seed=61, kind="ties", masked=0.05, nans=0.05, zeros=0.1)
    lens = [0, 1, 63, 2047, 2048, 2049, 9000, 12000, -5]
    for ld, off in ((9000, 0), (9013, 0), (9000, 1), (9016, 4)):
        print(f"[topk] ragged ld={ld} offset={off}", flush=True)
        got = _run(s, 2048, lens=lens, ld=ld, offset=off)
        ref = topk_general(s, 2048, row_lens=lens)
        assert np.array_equal(got, ref), (ld, off)


def test_topk_general_empty_rows_and_n0():
    s = np.zeros((3, 0), dtype=np.float32)
    got = _run(s, 5)
    assert np.all(got == -1)
    out = torch.empty((0, 5), dtype=torch.int32, device="cuda")
    dsa.dsa_topk(None, 0, 10, 10, None, 5, out)   # no rows: a no-op


def test_topk_general_deterministic():
    s = gen.make_topk_scores(64, 50000, seed=62, kind="ties", masked=0.02)
    a, b = _run(s, 2048), _run(s, 2048)
    assert np.array_equal(a, b)


def test_topk_general_full_workload_sampled():
    """The benchmark workload (2048 rows x 131072), in the launch the benchmark times; rows
    sampled for the oracle."""
    w = workloads.WORKLOADS[workloads.TOPK]
    s = workloads.make(workloads.TOPK)
    dev = torch.from_numpy(s).cuda()
    out = torch.empty((w["rows"], w["topk"]), dtype=torch.int32, device="cuda")
    dsa.dsa_topk(dev, w["rows"], w["n"], w["n"], None, w["topk"], out)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 777, 1024, 2047])
    got = out[torch.from_numpy(rows).cuda()].cpu().numpy()
    assert np.array_equal(got, topk_general(s[rows], w["topk"]))
