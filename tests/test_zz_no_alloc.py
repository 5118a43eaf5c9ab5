"""w4_linear_noalloc (the layer with the library's own device scratch instead
of a workspace argument) against w4_linear on the same inputs, through the C
ABI: identical outputs (same kernels, same fixed sum order), and within the
oracle's tolerance, on consecutive calls whose scratch use shrinks (the
array keeps the previous call's contents)."""
import numpy as np
import pytest
import torch

import oracle as O
from int4_weight_quantized_amd import ops
from int4_weight_quantized_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _dev_half(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).to(DEV)


def _layer(M, K, N, group, dtype, seed):
    d = W.w4a8_inputs(M, K, N, group, dtype, seed=seed, with_bias=True)
    wt = ops.w4_repack(torch.from_numpy(d["qweight"]).to(DEV), ops.W4_LAYOUT_GPTQ_KN, K, N)
    sc = torch.from_numpy(np.ascontiguousarray(d["scales"])).to(DEV)
    return d, _dev_half(d["x"], dtype), wt, sc, _dev_half(d["bias"], dtype)


@pytest.mark.parametrize("calls", [
    # (M, K, N, group, dtype): the first two take the int8 path with K split
    # (codes, row scales and fp32 partial tiles in the scratch), the second
    # smaller; then an unsplit int8 call and a weight-only one
    [(64, 1024, 2056, 128, "bf16"), (40, 1024, 1032, 128, "bf16"), (300, 1152, 520, 384, "f16"),
     (8, 1024, 264, 128, "bf16")],
    [(4096, 4096, 1024, 128, "bf16"), (48, 2048, 528, -1, "f16")],
])
def test_noalloc_matches_w4_linear(calls):
    for i, (M, K, N, group, dtype) in enumerate(calls):
        print(f"\n[noalloc] call {i}: M={M} K={K} N={N} group={group} {dtype}", flush=True)
        d, x, wt, sc, b = _layer(M, K, N, group, dtype, seed=1000 + 17 * i + M)
        need = ops.w4_linear_workspace_bytes(M, N, K, group)
        assert need <= ops.W4_LINEAR_NOALLOC_SCRATCH_BYTES
        y_ref = ops.w4_linear(x, wt, sc, group, N, bias=b)
        y = ops.w4_linear_noalloc(x, wt, sc, group, N, bias=b)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"call {i}: noalloc output differs from w4_linear"
        rows = np.arange(M) if M <= 64 else np.sort(np.random.default_rng(i).choice(M, 48, replace=False))
        if M < ops.W4_LINEAR_MIN_TOKENS_INT8:
            ref = O.w4a16_gptq_reference(d["x"], dtype, d["qweight"], d["scales"], group, bias_bits=d["bias"])
        else:
            ref = O.w4a8_reference(d["x"], dtype, d["qweight"], d["scales"], group, bias_bits=d["bias"],
                                   rows=rows)["y"]
        g = y[torch.from_numpy(rows).to(DEV)] if M >= ops.W4_LINEAR_MIN_TOKENS_INT8 else y
        err = np.abs(g.float().cpu().numpy().astype(np.float64) - ref) - (1e-3 + 1e-2 * np.abs(ref))
        assert err.max() <= 0, f"call {i}: outside 1e-3 + 1e-2|y| by {err.max():.3e}"
