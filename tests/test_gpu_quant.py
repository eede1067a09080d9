"""Quantised weight streaming against the oracle.

decoder_init turns every layer matrix and the lm-head into int8 codes with
one power-of-two scale per row; the model then computes with the
dequantised weights on every path.  The codes are integers, so the kernel's
must equal the oracle's bit for bit (and so must the dequantised bf16
weights, which are exact).  End to end, the quantised model's prefill and
teacher-forced decode meet the acceptance rule against the oracle run on
the same quantised weights.
"""
import numpy as np
import pytest

import oracle
import synth
from synth.weights import host_weights, prompt
from synth.workloads import C8B, TINY
from tests.gpu_util import assert_parity, compare_logits, decode, log, make_decoder, run_prefill

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("rows,K,sigma", [(37, 4096, 0.02), (8, 1000, 3.0), (5, 64, 1e-3)])
def test_quantize_kernel_bit_exact(rows, K, sigma):
    from decoder_only_transformer_step_amd.binding import diag_quantize_rows
    W = synth.normal_bf16(rows * K, 900 + rows, sigma).reshape(rows, K)
    W[0, :] = 0                                           # an all-zero row: scale 1, codes 0
    W[1, 3] = 0x8000                                      # a negative zero
    want_deq, want_e = oracle.quantize_rows(W, rows, K)
    dW = torch.from_numpy(W.view(np.int16)).cuda()
    q = torch.empty((rows, K), dtype=torch.int8, device="cuda")
    sc = torch.empty(rows, dtype=torch.float32, device="cuda")
    deq = torch.empty((rows, K), dtype=torch.int16, device="cuda")
    diag_quantize_rows(dW, rows, K, q, sc, deq, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got_deq = deq.cpu().numpy().view(np.uint16)
    got_q = q.cpu().numpy().astype(np.int64)
    got_s = sc.cpu().numpy()
    assert np.array_equal(got_s, np.ldexp(np.float32(1.0), want_e).astype(np.float32))
    want_q = np.rint(synth.bf16_to_f32(want_deq).astype(np.float64) / np.ldexp(1.0, want_e)[:, None])
    assert np.array_equal(got_q, want_q.astype(np.int64))
    # dequantised weights: equal values (a zero code may carry either sign)
    assert np.array_equal(synth.bf16_to_f32(got_deq), synth.bf16_to_f32(want_deq))


@pytest.mark.parametrize("rows,K,sigma", [(37, 4096, 0.02), (8, 1024, 3.0), (5, 64, 1e-3), (3, 14336, 0.02)])
def test_quantize_q4_kernel_bit_exact(rows, K, sigma):
    """4-bit codes, group exponents and dequantised weights equal the
    oracle's bit for bit (an all-zero group, a negative zero, groups whose
    largest magnitude sits exactly on 7 * 2^e)."""
    from decoder_only_transformer_step_amd.binding import diag_quantize_q4
    W = synth.normal_bf16(rows * K, 950 + rows, sigma).reshape(rows, K)
    W[0, :32] = 0                                         # an all-zero group: exponent 0, codes 0
    W[1, 3] = 0x8000                                      # a negative zero
    W[2, 32:64] = synth.f32_to_bf16(0.0)
    W[2, 40] = synth.f32_to_bf16(7.0 * 2.0 ** -6)         # largest magnitude exactly 7 * 2^-6
    W[2, 41] = synth.f32_to_bf16(-3.5 * 2.0 ** -6)        # code -3.5 -> -4 (ties to even)
    want_deq, want_q, want_e = oracle.quantize_q4(W, rows, K)
    assert want_e[2, 1] == -6 and want_q[2, 40] == 7 and want_q[2, 41] == -4
    dW = torch.from_numpy(W.view(np.int16)).cuda()
    codes = torch.empty((rows, K // 2), dtype=torch.uint8, device="cuda")
    exps = torch.empty((rows, K // 32), dtype=torch.int8, device="cuda")
    deq = torch.empty((rows, K), dtype=torch.int16, device="cuda")
    diag_quantize_q4(dW, codes, exps, deq, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    c = codes.cpu().numpy()
    got_q = np.empty((rows, K), np.int64)
    got_q[:, 0::2] = (c & 0xF).astype(np.int64) - 8
    got_q[:, 1::2] = (c >> 4).astype(np.int64) - 8
    assert np.array_equal(got_q, want_q.astype(np.int64))
    assert np.array_equal(exps.cpu().numpy().astype(np.int32), want_e)
    got_deq = deq.cpu().numpy().view(np.uint16)
    assert np.array_equal(synth.bf16_to_f32(got_deq), synth.bf16_to_f32(want_deq))


@pytest.mark.parametrize("N,K", [(16, 32), (100, 4096), (777, 2080), (4096, 14336)])
def test_gemv_q4_matches_oracle(N, K):
    """The batch-1 projection on 4-bit codes against the oracle's product
    with the dequantised weights (fp32 accumulation bound)."""
    from decoder_only_transformer_step_amd.binding import diag_gemv_q4, diag_quantize_q4
    log("gemv q4", N, K)
    W = synth.normal_bf16(N * K, 77 + N, 0.02).reshape(N, K)
    a = np.random.default_rng(N + K).normal(size=K).astype(np.float32)
    deq_h, _, e_h = oracle.quantize_q4(W, N, K)
    st = torch.cuda.current_stream().cuda_stream
    dW = torch.from_numpy(W.view(np.int16)).cuda()
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
    exps = torch.empty((N, K // 32), dtype=torch.int8, device="cuda")
    deq = torch.empty((N, K), dtype=torch.int16, device="cuda")
    diag_quantize_q4(dW, codes, exps, deq, st)
    y = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    diag_gemv_q4(torch.from_numpy(a).cuda(), codes, exps, y, st)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    want = oracle.matmul(deq_h, N, K, a.astype(np.float64)[None])[0]
    scale = np.abs(synth.bf16_to_f32(deq_h).astype(np.float64).reshape(N, K)) @ np.abs(a.astype(np.float64))
    # fp32 sums of exact products; the code offset adds 8 |sum of the group's activation| per group
    gsum = np.abs(a.astype(np.float64).reshape(-1, 32).sum(axis=1))
    off = (np.ldexp(1.0, e_h) * 8 * gsum[None, :]).sum(axis=1)
    assert np.all(np.abs(got - want) <= 1e-6 * np.sqrt(K) * (scale + off) + 1e-30)


SHAPES = {
    "tiny": (TINY.with_(name="gqa-tiny-q8", weight_quant=1), 16, 16, 8),
    "8b2": (C8B.with_(name="gqa-8b-layers-2-q8", n_layers=2, vocab=1024, max_seq=512, weight_quant=1),
            200, 128, 6),
    "tiny-q4": (TINY.with_(name="gqa-tiny-q4", ffn_inter=704, weight_quant=2), 16, 16, 8),
    "8b2-q4": (C8B.with_(name="gqa-8b-layers-2-q4", n_layers=2, vocab=1024, max_seq=512, weight_quant=2),
               200, 128, 6),
}


@pytest.mark.parametrize("which", ["tiny", "8b2", "tiny-q4", "8b2-q4"])
def test_quantized_model_prefill_and_decode(which):
    shape, P, chunk, steps = SHAPES[which]
    W = host_weights(shape)
    ids = prompt(shape, P)
    m = oracle.Model(shape, W)
    want = m.prefill(ids, chunk)["logits"]
    plain = oracle.Model(shape.with_(weight_quant=0), W).prefill(ids, chunk)["logits"]
    assert np.abs(plain - want).max() > 1e-3            # the quantisation moves the model
    dec, _ = make_decoder(shape, W)
    got = run_prefill(dec, ids, chunk)
    st = compare_logits(got, want, f"{which} q8 prefill")
    log(which, "q8 prefill", st)
    assert_parity(st, f"{which} q8 prefill")
    for i in range(steps):
        t = oracle.argmax(want)
        want = m.forward([t], P + i)["logits"]
        lg, _ = decode(dec, [0], [t])
        st = compare_logits(lg[0], want, f"{which} q8 decode {i}")
        log(which, "q8 decode", i, st)
        assert_parity(st, f"{which} q8 decode {i}")
    dec.close()


@pytest.mark.parametrize("bits", [8, 4])
def test_quantized_moe_prefill_decode_and_routes(bits):
    """int8 routed and shared experts (the grouped expert GEMV streams each
    chosen expert's codes with that expert's row scales): the small MoE
    model's logits against the oracle on the same quantised weights, and its
    expert ids layer by layer on the GPU's own router input."""
    from tests.moe_routes import check_routes_exact, forced
    from tests.test_gpu_parity import small_moe
    shape = small_moe().with_(name=f"moe-small-q{bits}", weight_quant=1 if bits == 8 else 2)
    W = host_weights(shape)
    ids = [int(t) for t in prompt(shape, 24)]
    m = oracle.Model(shape, W)
    plain = oracle.Model(shape.with_(weight_quant=0), W).forward(ids, 0)["logits"]
    dec, _ = make_decoder(shape, W)
    logits = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")

    def prefill():
        dec.kv_truncate(0, 0)
        dec.prefill_chunk(0, ids, 0, logits_mode=1, logits=logits)

    prefill()
    torch.cuda.synchronize()
    want = m.forward(ids, 0, force_routes=forced(dec, shape, 24))
    assert np.abs(plain - want["logits"]).max() > 1e-3
    st = compare_logits(logits.cpu().numpy(), want["logits"], "moe q8 prefill")
    log("moe q8 prefill", st)
    assert_parity(st, "moe q8 prefill")
    check_routes_exact(dec, shape, W, 24, prefill, "moe q8 prefill")
    for step in range(4):
        t = oracle.argmax(want["logits"])
        lg, _ = decode(dec, [0], [t])
        want = m.forward([t], 24 + step, force_routes=forced(dec, shape, 1))
        st = compare_logits(lg[0], want["logits"], f"moe q8 decode {step}")
        log("moe q8 decode", step, st)
        assert_parity(st, f"moe q8 decode {step}")
        check_routes_exact(dec, shape, W, 1, lambda: (dec.kv_truncate(0, 24 + step), decode(dec, [0], [t])),
                           f"moe q8 decode {step}")
    dec.close()


def test_quantized_moe_verify_streams_codes():
    """A 4-position verify pass of the small MoE model with int8 experts: the
    grouped expert projections of a pass of at most 16 rows stream each
    chosen expert's int8 codes with its row scales.  Every row's logits meet
    the acceptance rule against the oracle (which follows the GPU's expert
    ids), and those ids are exact on the GPU's own router input."""
    from tests.moe_routes import check_routes_exact, forced
    from tests.test_gpu_parity import small_moe
    shape = small_moe().with_(name="moe-small-q8", weight_quant=1)
    W = host_weights(shape)
    ids = [int(t) for t in prompt(shape, 28, seq=4)]
    m = oracle.Model(shape, W)
    dec, _ = make_decoder(shape, W)
    dec.prefill_chunk(0, ids[:24], 0, logits_mode=0)
    torch.cuda.synchronize()
    m.forward(ids[:24], 0, logits_mode=0, force_routes=forced(dec, shape, 24))
    logits = torch.empty((4, shape.vocab), dtype=torch.float32, device="cuda")

    def verify():
        dec.kv_truncate(0, 24)
        dec.prefill_chunk(0, ids[24:], 24, logits_mode=2, logits=logits)

    verify()
    torch.cuda.synchronize()
    want = m.forward(ids[24:], 24, logits_mode=2, force_routes=forced(dec, shape, 4))["logits"]
    got = logits.cpu().numpy()
    for i in range(4):
        st = compare_logits(got[i], want[i], f"moe q8 verify row {i}")
        log("moe q8 verify row", i, st)
        assert_parity(st, f"moe q8 verify row {i}")
    check_routes_exact(dec, shape, W, 4, verify, "moe q8 verify")
    dec.close()
