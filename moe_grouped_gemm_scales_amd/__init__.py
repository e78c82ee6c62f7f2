"""MI355X (gfx950) block-scaled FP8 GEMM: D = C + A.B^T in dense, M-grouped
contiguous and M-grouped masked forms (FP32 or UE8M0 scales, FP8 x FP4 and FP4 x FP4),
the NN/TN/TT storage layouts, the K-grouped TN form and an unscaled BF16 GEMM,
as a C-ABI library (libdg.so) with a thin Python binding.  See include/dg.h
for the contract."""
from .dg import get_wait_giveups, reset_wait_giveups  # noqa: F401
from .dg import (SCALE_UE8M0_I16, dg_fp8_gemm_nt_ue8m0_i16, dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0_i16,  # noqa: F401
                 dg_m_grouped_fp8_gemm_nt_masked_ue8m0_i16)
from .dg import (DGError, describe_config, dg_fp8_gemm_nt, dg_m_grouped_fp8_gemm_nt_contiguous,  # noqa: F401
                 dg_m_grouped_fp8_gemm_nt_masked, fp8_gemm_nt, get_mk_alignment_for_contiguous_layout,
                 get_num_cus, init, m_grouped_fp8_gemm_nt_contiguous, m_grouped_fp8_gemm_nt_masked,
                 precompile, set_num_cus, SCALE_UE8M0, dg_fp8_gemm_nt_ue8m0,
                 dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0, dg_m_grouped_fp8_gemm_nt_masked_ue8m0,
                 SCALE_FP8_FP4, dg_fp8_fp4_gemm_nt, dg_m_grouped_fp8_fp4_gemm_nt_contiguous,
                 dg_m_grouped_fp8_fp4_gemm_nt_masked, fp8_fp4_gemm_nt, m_grouped_fp8_fp4_gemm_nt_contiguous,
                 m_grouped_fp8_fp4_gemm_nt_masked, KIND_K_GROUPED, dg_k_grouped_fp8_gemm_tn_contiguous,
                 k_grouped_fp8_gemm_tn_contiguous, dg_fp8_gemm_nn, dg_fp8_gemm_tn, dg_fp8_gemm_tt,
                 dg_m_grouped_fp8_gemm_nn_contiguous, fp8_gemm_nn, fp8_gemm_tn, fp8_gemm_tt,
                 m_grouped_fp8_gemm_nn_contiguous, KIND_BF16, dg_bf16_gemm_nt,
                 dg_m_grouped_bf16_gemm_nt_contiguous, dg_m_grouped_bf16_gemm_nt_masked, bf16_gemm_nt,
                 m_grouped_bf16_gemm_nt_contiguous, m_grouped_bf16_gemm_nt_masked, SCALE_FP4_FP4,
                 dg_fp4_fp4_gemm_nt, dg_m_grouped_fp4_fp4_gemm_nt_contiguous, dg_m_grouped_fp4_fp4_gemm_nt_masked,
                 fp4_fp4_gemm_nt, m_grouped_fp4_fp4_gemm_nt_contiguous, m_grouped_fp4_fp4_gemm_nt_masked)
