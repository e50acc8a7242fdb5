"""gptq_accumulate_hessian_noalloc (the Hessian accumulation for callers that
cannot allocate: split-K partials in the library's static device array, X
read token-major) against gptq_accumulate_hessian with a caller workspace,
through the C ABI. The shapes are narrower than the width where the
workspace form switches to a feature-major copy of X (d >= 12288), so both
run the same kernels and plan, and H must agree bit for bit. Two calls in a row,
the second smaller (the array keeps the first call's partials), on shapes
that use the token-split partials (d = 2560), the stream-K partials
(d = 4352) and a small token split (d = 256, 1024 tokens); then a size beyond the
array is rejected before anything is enqueued."""

import ctypes

import pytest
import torch

from post_weight_quantization_18_amd import gptq as G
from post_weight_quantization_18_amd import synthetic as S

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _noalloc(H, X, accumulate):
    lib = G.load_library()
    d, n = H.shape[0], X.shape[0]
    return lib.gptq_accumulate_hessian_noalloc(G._ptr(H), G._DT[H.dtype], d, H.stride(0), G._ptr(X), n, X.stride(0),
                                               int(accumulate), G._stream(DEV))


@pytest.mark.parametrize("d,n", [(2560, 65536), (4352, 40960), (256, 1024)])
def test_noalloc_matches_workspace_entry_point(d, n):
    print(f"[case] noalloc d={d} n={n} then n/2, d/2", flush=True)
    cfg = S.scaled(S.CONFIGS["opt13b-attn"], m=64, d=d, n_tokens=n)
    x = S.make_activations(cfg, DEV)
    for (dd, nn) in ((d, n), (d // 2, n // 2)):
        xs = x[:nn, :dd].contiguous()
        ws = torch.empty(max(1, G.workspace_bytes(G.WS_ACCUMULATE_HESSIAN, 0, dd, nn)), dtype=torch.uint8,
                         device=DEV)
        for h_dtype in (torch.float64, torch.float32):
            ref = torch.empty(dd, dd, dtype=h_dtype, device=DEV)
            G.accumulate_hessian(ref, xs, accumulate=False, workspace=ws)
            got = torch.full((dd, dd), float("nan"), dtype=h_dtype, device=DEV)
            assert _noalloc(got, xs, False) == G.GPTQ_OK
            # then accumulate a second pass onto it, as a streaming caller would
            G.accumulate_hessian(ref, xs, accumulate=True, workspace=ws)
            assert _noalloc(got, xs, True) == G.GPTQ_OK
            torch.cuda.synchronize()
            lo = torch.tril(torch.ones(dd, dd, dtype=torch.bool, device=DEV))
            assert torch.equal(got[lo], ref[lo]), (dd, nn, h_dtype)
            assert torch.isnan(got[~lo]).all()  # the strictly upper triangle is not touched


def test_noalloc_rejects_sizes_beyond_the_array():
    print("[case] noalloc too large", flush=True)
    d, n = 3360, 1 << 19
    need = G.workspace_bytes(G.WS_ACCUMULATE_HESSIAN, 0, d, n)
    assert need > 192 << 20
    H = torch.empty(d, d, dtype=torch.float64, device=DEV)
    X = torch.empty(8, d, dtype=torch.float16, device=DEV)  # never read: the call is rejected first
    lib = G.load_library()
    st = lib.gptq_accumulate_hessian_noalloc(G._ptr(H), G.GPTQ_F64, d, d, G._ptr(X), n, d, 0, G._stream(DEV))
    assert st == G.GPTQ_ERR_WORKSPACE
