"""full_vocab_kl_amd -- libkld, full-vocabulary KL scoring on AMD MI355X.

The compute lives in the C-ABI library ``libkld.so`` (hand-written HIP for
gfx950, declared in include/kld.h).  ``full_vocab_kl_amd.binding`` is a thin
ctypes binding with the same entry-point names; it only marshals torch
device tensors and the current HIP stream into the C calls and raises if
the library is not built."""
from .binding import (  # noqa: F401
    KldError, KLD_F32, KLD_BF16, TOPK, lib, library_path, kld_workspace_size, kld_from_logits,
    kld_fused_head, topk_export, kld_topk_tail, kld_summary, summary_dict, kld_status_str,
    kld_abi_version, GOLDEN_TOPK, kld_golden_export, kld_coarse_kl,
    kld_window_summary, kld_paired_bootstrap, kld_coarse_fused, kld_from_logits_noalloc,
)
