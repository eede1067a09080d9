"""dec_diag_gemm_chunk_noalloc: the chunk projection with its split-K
partials in the library's static per-device array (no workspace argument,
no allocation).  Its output must equal dec_diag_gemm_chunk's on the same
inputs (same kernels, same split, same fixed reduction order: bit for bit)
and meet the oracle's bound, on two calls in a row, the second smaller, so
the second reads nothing the first left behind."""
import numpy as np
import pytest

import oracle
import synth
from decoder_only_transformer_step_amd import binding
from tests.gpu_util import log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def bits_of(x):
    return synth.bf16_to_f32(x)


def run_pair(M, N, K, ksplit, seed):
    from decoder_only_transformer_step_amd.binding import diag_gemm_chunk, diag_gemm_chunk_noalloc, diag_pack_w32
    st = torch.cuda.current_stream().cuda_stream
    hi = synth.normal_bf16(M * K, seed, 1.0)
    lo = synth.normal_bf16(M * K, seed + 1, 2.0 ** -9)
    A = np.stack([hi, lo])
    W = synth.normal_bf16(N * K, seed + 2, 0.02)
    dA = torch.from_numpy(A.view(np.int16)).cuda().view(2, M, K)
    dW = torch.from_numpy(W.view(np.int16)).cuda().view(N, K)
    dP = torch.empty_like(dW)
    diag_pack_w32(dW, dP, st)
    ref = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    part = torch.full((ksplit * M * N,), float("nan"), dtype=torch.float32, device="cuda")
    diag_gemm_chunk(dA, dP, ref, ksplit, part, st)
    got = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    diag_gemm_chunk_noalloc(dA, dP, got, ksplit, st)
    torch.cuda.synchronize()
    ref, got = ref.cpu().numpy(), got.cpu().numpy()
    assert np.array_equal(got, ref), (M, N, K, ksplit)
    a = sum(bits_of(A[p]).astype(np.float64).reshape(M, K) for p in range(2))
    want = oracle.matmul(W, N, K, a)
    scale = sum(np.abs(bits_of(A[p]).astype(np.float64).reshape(M, K)) for p in range(2)) @ \
        np.abs(bits_of(W)).reshape(N, K).T.astype(np.float64)
    assert np.all(np.abs(got.astype(np.float64) - want) <= 1e-6 * K * scale + 1e-30)
    log("noalloc", M, N, K, ksplit, "equal to the workspace entry point and within the oracle bound")


def test_noalloc_matches_workspace_entry_point_twice():
    run_pair(128, 4096, 4096, 8, 101)     # 8 x 128 x 4096 = 4 Mi partial floats: the whole array
    run_pair(37, 96, 688, 3, 211)         # smaller, ragged: reads only what it wrote


def test_noalloc_refuses_partials_beyond_its_array():
    # 9 x 128 x 4096 partial floats exceed the 4 Mi the array holds
    M, N, K = 128, 4096, 4096
    dA = torch.zeros((2, M, K), dtype=torch.int16, device="cuda")
    dP = torch.zeros((N, K), dtype=torch.int16, device="cuda")
    C = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    rc = binding.lib().dec_diag_gemm_chunk_noalloc(binding._ptr(dA), 2, M, K, binding._ptr(dP), N,
                                                   binding._ptr(C), 9, None)
    assert rc == binding.DEC_E_WORKSPACE
    torch.cuda.synchronize()
