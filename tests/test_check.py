"""Negative controls for the acceptance check (tests/check.py): outputs with a
plausible kernel mistake must be rejected, and outputs that differ from the
oracle only by FP32 summation order and BF16 rounding must be accepted.  CPU
only; the "kernel outputs" here are computed with the oracle or numpy."""
import numpy as np
import torch

from tests import check, gen


def _bf16_round(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy() \
        .astype(np.float64)


def _problem():
    # N = 2112: the last 128-row block of B has 64 rows (the first workload's tail)
    return gen.make_dense(16, 2112, 1024, seed=77, with_c=False)


def test_correct_and_reordered_outputs_pass(oracle):
    p = _problem()
    ref = oracle.fp8_gemm_nt(p.A.numpy(), p.sfa.numpy(), p.B.numpy(), p.sfb.numpy())
    assert check.within_tolerance(_bf16_round(ref), ref)[0]
    # FP32 dequantise-and-matmul (another summation order), then BF16
    dec = p.A.view(torch.float8_e4m3fn).float() * p.sfa.t().repeat_interleave(128, 1)
    sb = p.sfb.repeat_interleave(128, 0)[:2112].repeat_interleave(128, 1)
    decb = p.B.view(torch.float8_e4m3fn).float() * sb
    got = (dec @ decb.t()).numpy()
    assert check.within_tolerance(_bf16_round(got), ref)[0]


def test_dropped_last_k_block_is_rejected(oracle):
    p = _problem()
    ref = oracle.fp8_gemm_nt(p.A.numpy(), p.sfa.numpy(), p.B.numpy(), p.sfb.numpy())
    A = p.A.numpy().copy()
    A[:, -128:] = 0                       # E4M3 +0: the last K block contributes nothing
    wrong = oracle.fp8_gemm_nt(A, p.sfa.numpy(), p.B.numpy(), p.sfb.numpy())
    assert not check.within_tolerance(_bf16_round(wrong), ref)[0]


def test_fnuz_decoding_is_rejected(oracle):
    """E4M3FNUZ reads the same bits with exponent bias 8: every normal value halves."""
    p = _problem()
    ref = oracle.fp8_gemm_nt(p.A.numpy(), p.sfa.numpy(), p.B.numpy(), p.sfb.numpy())
    wrong = oracle.fp8_gemm_nt(p.A.numpy(), (p.sfa * 0.5).numpy(), p.B.numpy(), (p.sfb * 0.5).numpy())
    assert not check.within_tolerance(_bf16_round(wrong), ref)[0]


def test_wrong_scale_block_at_the_n_tail_is_rejected(oracle):
    p = _problem()
    ref = oracle.fp8_gemm_nt(p.A.numpy(), p.sfa.numpy(), p.B.numpy(), p.sfb.numpy())
    sfb = p.sfb.numpy().copy()
    sfb[16] = sfb[15]                     # columns 2048..2111 scaled with the previous block
    assert not np.allclose(sfb[16], p.sfb.numpy()[16])
    wrong = oracle.fp8_gemm_nt(p.A.numpy(), p.sfa.numpy(), p.B.numpy(), sfb)
    assert not check.within_tolerance(_bf16_round(wrong), ref)[0]


def test_ignored_c_and_one_wrong_element_are_rejected(oracle):
    p = gen.make_dense(16, 256, 512, seed=78, with_c=True)
    ref = oracle.fp8_gemm_nt(p.A.numpy(), p.sfa.numpy(), p.B.numpy(), p.sfb.numpy(), p.C.numpy())
    no_c = oracle.fp8_gemm_nt(p.A.numpy(), p.sfa.numpy(), p.B.numpy(), p.sfb.numpy())
    assert not check.within_tolerance(_bf16_round(no_c), ref)[0]
    one = _bf16_round(ref)
    one[7, 100] = -one[7, 100] + 1.0      # a single element off
    assert not check.within_tolerance(one, ref)[0]


def test_written_masked_row_is_detected():
    """Untouched rows are compared bit for bit with their sentinel prefill."""
    sent = gen.sentinel_like((4, 64), 5)
    out = sent.clone()
    assert np.array_equal(check.bf16_bits(out), check.bf16_bits(sent))
    out[2, 10] = torch.tensor(0.0, dtype=torch.bfloat16)
    assert not np.array_equal(check.bf16_bits(out), check.bf16_bits(sent))
