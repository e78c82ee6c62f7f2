"""The bench's FLOP and byte convention reproduces the pages' own table: with
t = 2MNK / TFLOPS, (|A| + |B| + |D|) / t (1-byte A and B, 2-byte D) gives the
GB/s column of the DeepGEMM launch article's dense table (tests/golden)."""
import json
import os

import torch

import bench
from tests import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_benchmarks.json")


def test_pages_gbs_follow_from_their_tflops():
    rows = json.load(open(GOLDEN))["rows"]
    for r in rows:
        M, N, K = r["M"], r["N"], r["K"]
        # a dense problem of that shape, built without data (only sizes matter)
        p = gen.Problem("dense", torch.empty(M, K, dtype=torch.uint8), torch.empty(K // 128, M),
                        torch.empty(N, K, dtype=torch.uint8), torch.empty((N + 127) // 128, K // 128))
        flops, nbytes, rows_ = bench.algorithmic(p)
        assert flops == 2.0 * M * N * K and rows_ == M
        t = flops / (r["tflops"] * 1e12)
        scales = M * (K // 128) * 4 + ((N + 127) // 128) * (K // 128) * 4
        gbs = (nbytes - scales) / t / 1e9
        # the table's TFLOPS are rounded to integers: agree within that rounding
        assert abs(gbs - r["gbs"]) / r["gbs"] < 0.005, (r, gbs)


def test_roofline_bound_classification():
    # ridge point of 5.0 PFLOP/s over 8 TB/s: 625 FLOP/byte
    assert abs(bench.RIDGE - 625.0) < 1e-9
    for cfg, bound in [(0, "hbm"), (1, "hbm"), (2, "mfma")]:
        c = gen.WORKLOADS[cfg]
        M, N, K = c["M"], c["N"], c["K"]
        p = gen.Problem("dense", torch.empty(M, K, dtype=torch.uint8), torch.empty(K // 128, M),
                        torch.empty(N, K, dtype=torch.uint8), torch.empty((N + 127) // 128, K // 128))
        flops, nbytes, _ = bench.algorithmic(p)
        assert ("mfma" if flops / nbytes >= bench.RIDGE else "hbm") == bound
