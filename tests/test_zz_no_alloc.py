"""nf_op_gemm_noalloc (the allocation-free entry point) against nf_op_gemm, through the C ABI.

Split-K products keep their fp32 partials in the library's static scratch instead of the
context's workspace; the results must be those of nf_op_gemm (the same kernels, the same
summation order: bitwise equal), on consecutive calls of decreasing size, and a product
whose partials exceed the scratch is refused before anything is enqueued.
"""

import numpy as np
import pytest

from tests.gpu_util import log_case, rand_bf16

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

# (m, n, k, epilogue, variant): split-K configurations, largest first (the first one's
# partials, 2 x 2048 x 4096 x 4 bytes, fill the 64 MiB scratch exactly)
CASES = [
    (2048, 4096, 14336, 1, 25),  # 256x256, 2 K slices: the 8B Down product
    (1024, 4096, 14336, 1, -1),  # the library's choice for a 1024-row nano-batch (K in 4 slices)
    (300, 688, 4096, 0, 10),     # 128x128, 2 K slices, ragged tiles
    (77, 520, 4096, 1, 11),      # 128x128, 4 K slices, ragged tiles, residual
]


def _dev(bits):
    from nano_intra_overlap_amd.device import bf16_tensor

    return bf16_tensor(bits, "cuda")


def test_noalloc_gemm_matches_nf_op_gemm():
    from nano_intra_overlap_amd import abi
    from nano_intra_overlap_amd.device import bf16_bits

    ctx_ref = abi.nf_ctx_create(0)
    ctx = abi.nf_ctx_create(0)
    stream = torch.cuda.current_stream().cuda_stream
    try:
        data = []
        for m, n, k, epi, v in CASES:
            assert abi.nf_gemm_choice(m, n, k, epi)[1]
            if v >= 0:
                assert abi.nf_gemm_variants()[v][3] > 1, "a split-K configuration"
            else:
                assert abi.nf_gemm_variants()[abi.nf_gemm_choice(m, n, k, epi)[0]][3] > 1
            rng = np.random.default_rng(m + n + k + epi)
            A, B, R = (_dev(rand_bf16(rng, (m, k))), _dev(rand_bf16(rng, (n, k), 0.05)),
                       _dev(rand_bf16(rng, (m, n))))
            data.append((A, B, R, torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda"),
                         torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")))
        # a product whose partials exceed the scratch: refused, output untouched
        big_A = torch.zeros((2048, 8192), dtype=torch.bfloat16, device="cuda")
        big_B = torch.zeros((8192, 8192), dtype=torch.bfloat16, device="cuda")
        big_C = torch.full((2048, 8192), float("nan"), dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()

        def device_memory_not_torch():
            # free device memory plus what torch's caching allocator holds: changes only when
            # something other than torch allocates or frees device memory
            return torch.cuda.mem_get_info()[0] + torch.cuda.memory_reserved()

        free0 = None
        for rnd in range(2):  # the same sequence twice: the scratch keeps the last call's contents
            for (m, n, k, epi, v), (A, B, R, C_ref, C) in zip(CASES, data):
                log_case(f"noalloc gemm round {rnd} m={m} n={n} k={k} epi={epi} variant={v}")
                C_ref.fill_(float("nan"))
                C.fill_(float("nan"))
                abi.nf_op_gemm(ctx_ref, A.data_ptr(), B.data_ptr(), C_ref.data_ptr(), R.data_ptr(), m, n, k, epi, v,
                               stream)
                abi.nf_op_gemm_noalloc(ctx, A.data_ptr(), B.data_ptr(), C.data_ptr(), R.data_ptr(), m, n, k, epi, v,
                                       stream)
                torch.cuda.synchronize()
                got, want = bf16_bits(C), bf16_bits(C_ref)
                assert not torch.isnan(C.float()).any()
                assert np.array_equal(got, want), (m, n, k, epi, v)
                if free0 is None:
                    free0 = device_memory_not_torch()
            log_case(f"noalloc gemm round {rnd}: oversized product refused")
            with pytest.raises(abi.NanoflowError) as e:
                abi.nf_op_gemm_noalloc(ctx, big_A.data_ptr(), big_B.data_ptr(), big_C.data_ptr(), None, 2048, 8192,
                                       8192, 0, 25, stream)
            assert e.value.status == abi.NF_E_CAPACITY
        torch.cuda.synchronize()
        assert torch.isnan(big_C.float()).all()
        # no device memory was taken by the allocation-free calls after the first
        assert device_memory_not_torch() >= free0, (free0, device_memory_not_torch())
    finally:
        abi.nf_ctx_destroy(ctx)
        abi.nf_ctx_destroy(ctx_ref)
