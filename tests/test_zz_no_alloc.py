"""GPU check of kld_from_logits_noalloc (the allocation-free variant for
callers that cannot allocate): through the C ABI it must give exactly the
outputs of kld_from_logits with a caller workspace, on two calls in a row,
the second with a smaller input (the static scratch keeps the first call's
contents)."""
import numpy as np
import pytest
import torch

import synth
import full_vocab_kl_amd as kld
from gpu_util import gpu, need_gpu, to_dev

pytestmark = gpu


def _outputs(n, dev, target):
    f = dict(dtype=torch.float32, device=dev)
    out = {"kl": torch.full((n,), float("nan"), **f), "lse_ref": torch.empty(n, **f),
           "lse_cand": torch.empty(n, **f),
           "argmax_ref": torch.full((n,), -7, dtype=torch.int32, device=dev),
           "argmax_cand": torch.full((n,), -7, dtype=torch.int32, device=dev),
           "ids_ref": torch.full((n, 64), -7, dtype=torch.int32, device=dev),
           "ids_cand": torch.full((n, 64), -7, dtype=torch.int32, device=dev),
           "lp_ref": torch.zeros((n, 64), dtype=torch.float16, device=dev),
           "lp_cand": torch.zeros((n, 64), dtype=torch.float16, device=dev)}
    if target is not None:
        out["nll_ref"] = torch.empty(n, **f)
        out["nll_cand"] = torch.empty(n, **f)
    return out


def _same(a, b, where):
    for k in a:
        x, y = a[k].cpu().numpy(), b[k].cpu().numpy()
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"{where}: {k} differs"


@pytest.mark.parametrize("first,second", [((600, 50_000, False, True), (37, 5003, True, False))])
def test_noalloc_matches_workspace_entry_point(first, second):
    dev = need_gpu()
    for n, v, bf16, with_target in (first, second):
        print(f"noalloc case n={n} v={v} bf16={bf16} target={with_target}", flush=True)
        a, b = synth.logit_rows(synth.LOGITS_BF16_TOPK, range(n), v)
        if bf16:
            a, b = synth.f32_to_bf16_bits(a), synth.f32_to_bf16_bits(b)
        ra, rb = to_dev(a, bf16), to_dev(b, bf16)
        t = to_dev(synth.targets(synth.LOGITS_BF16_TOPK, range(n), v)) if with_target else None
        want = kld.kld_from_logits(ra, rb, t, topk=True, out=_outputs(n, dev, t))
        got = kld.kld_from_logits_noalloc(ra, rb, t, topk=True, out=_outputs(n, dev, t))
        torch.cuda.synchronize()
        assert np.all(np.isfinite(got["kl"].cpu().numpy()))
        _same(want, got, f"n={n} v={v}")
