"""The allocation-free GEMM entry point (tern_gemm_noalloc) through the C ABI.

It runs the same kernels as tern_gemm with the K-split partial sums in the
library's static device scratch, so its output must equal tern_gemm's bit for
bit.  Two calls in a row, the second on a smaller problem, check that the
shared scratch left by the first call does not leak into the second; sampled
columns of each are also checked against the FP64 oracle.  A size whose
partial sums exceed the scratch is refused before any launch.
"""
import numpy as np
import pytest

import synth
from tests._helpers import assert_matmul_close, pack_to_device, sampled_rows, torch, x_to_device, y_to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tern():
    T = torch()
    if not T.cuda.is_available():
        pytest.skip("no GPU")
    import ternary_weight_g128_amd as t
    return t


def test_gemm_noalloc_matches_gemm_on_two_calls(tern, oracle_lib):
    T = torch()
    # both shapes split tiles along K on a 256-CU device, so both use the scratch
    for M, K, N in [(200, 2304, 4096), (100, 1536, 1280)]:
        seed = 3 * M + K + N
        need = tern.tern_gemm_workspace_bytes(M, N, K)
        print(f"gemm_noalloc M={M} K={K} N={N} scratch={need} seed={seed}", flush=True)
        assert 0 < need <= tern.TERN_GEMM_SCRATCH_BYTES, need
        t = synth.ternary(seed, N, K, 0.35)
        s = synth.scales_f16(seed, N, K)
        x = synth.activations_bf16(seed, M, K, outlier_frac=0.01)
        codes_d, scales_d = pack_to_device(tern, t, s)
        xd = x_to_device(x)
        y_ref = tern.tern_gemm(xd, codes_d, scales_d)
        y = T.full((M, N), float("nan"), dtype=T.float32, device="cuda")
        tern.tern_gemm_noalloc(xd, codes_d, scales_d, out=y)
        T.cuda.synchronize()
        assert T.equal(y, y_ref), f"M{M} K{K} N{N}: noalloc differs from tern_gemm"
        cols = sampled_rows(N, 24, seed)
        y_or, bound = oracle_lib.matmul(x, oracle_lib.encode(t[cols]), s[cols], K)
        assert_matmul_close(y_to_host(y)[:, cols], y_or, bound, what=f"gemm_noalloc M{M} K{K} N{N}")


def test_gemm_noalloc_refuses_sizes_beyond_the_scratch(tern):
    T = torch()
    M, K, N = 512, 17408, 12288
    need = tern.tern_gemm_workspace_bytes(M, N, K)
    print(f"gemm_noalloc refusal M={M} K={K} N={N} scratch={need}", flush=True)
    assert need > tern.TERN_GEMM_SCRATCH_BYTES, need
    # real buffers of the right shapes; the call must fail on the host
    x = T.empty((M, K), dtype=T.bfloat16, device="cuda")
    codes = T.empty((N, K // 16), dtype=T.int32, device="cuda")
    scales = T.empty((N, K // 128), dtype=T.int16, device="cuda")
    y = T.empty((M, N), dtype=T.float32, device="cuda")
    with pytest.raises(tern.TernError) as e:
        tern.tern_gemm_noalloc(x, codes, scales, out=y)
    assert e.value.status == tern.TERN_EUNSUPPORTED
    assert "TERN_GEMM_SCRATCH_BYTES" in str(e.value)
