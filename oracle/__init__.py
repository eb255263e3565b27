"""Plain f64 CPU oracle (test infrastructure only; see kld_oracle)."""
from .kld_oracle import (  # noqa: F401
    TOPK, bf16_bits_to_f64, fp16_bits_to_f64, f64_to_fp16_bits, logsumexp, kl_row,
    argmax_row, nll_row, topk_row, tail_kld_probs, tail_kld_row, head_logits, score_rows, percentile,
    summarize, GOLDEN_TOPK, golden_row, golden_rows, coarse_kl_row, coarse_kl_rows,
    window_summary, paired_bootstrap,
)
