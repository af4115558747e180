"""GPU: the allocation-free percentile (sq_calib_percentile_noalloc, its
scratch in a static device array of the library) gives what the workspace
form gives, on two calls in a row -- the second smaller, so it reuses the
array the first left dirty -- and refuses a problem past the array's size
before launching anything."""
from __future__ import annotations

import numpy as np
import pytest

from tests.gpu_pipeline import assert_bitexact, dev
from w8a8_post_quantization_channel_amd import capi, synth

pytestmark = pytest.mark.gpu


def _workspace_form(x, q):
    import torch
    k = x.shape[1]
    code = capi.SQ_BF16 if x.dtype == torch.bfloat16 else capi.SQ_F32
    ws = torch.empty(capi.sq_calib_percentile_workspace(k, code), dtype=torch.uint8, device=x.device)
    out = torch.empty(k, dtype=torch.float32, device=x.device)
    capi.sq_calib_percentile(x, q, ws, out)
    return out


def _noalloc(x, q):
    import torch
    out = torch.empty(x.shape[1], dtype=torch.float32, device=x.device)
    capi.sq_calib_percentile_noalloc(x, q, out)
    return out


def test_noalloc_percentile_matches_workspace_form():
    import torch
    d = dev()
    cases = [
        # (rows, k, q, bf16): the first fills most of the array's bf16 range, the second is smaller
        (65536, 13824, 0.999, True),
        (3000, 1024, 0.5, True),
        (4096, 8128, 0.9995, False),   # the largest fp32 width that fits
        (777, 192, 1.0, False),
    ]
    for i, (rows, k, q, bf16) in enumerate(cases):
        out = synth.outlier_channels(7100 + i, k)
        x = synth.to_torch(synth.activations(7200 + i, rows, k, out, bf16=bf16), d)
        got = _noalloc(x, q)
        ref = _workspace_form(x, q)
        torch.cuda.synchronize()
        assert_bitexact(f"case {i}", synth.from_torch(got), synth.from_torch(ref))
        assert np.all(np.isfinite(synth.from_torch(got)))


def test_noalloc_percentile_rejects_oversized():
    import torch
    d = dev()
    x = torch.zeros((64, 16384), dtype=torch.bfloat16, device=d)
    out = torch.full((16384,), 3.0, dtype=torch.float32, device=d)
    with pytest.raises(capi.SQError) as e:
        capi.sq_calib_percentile_noalloc(x, 0.5, out)
    assert e.value.status == 8
    torch.cuda.synchronize()
    assert float(out.max().item()) == 3.0 and float(out.min().item()) == 3.0  # nothing written
