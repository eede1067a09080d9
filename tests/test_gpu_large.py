"""GPU-vs-oracle parity at the workloads' full model sizes.

The oracle runs bounded slices of each workload (it finishes them in
seconds to tens of seconds on the host cores): the 135M-class model over its
whole prompt plus decode steps, the 8B-class model over one full 128-token
chunk plus decode steps, the 60-expert MoE over one chunk plus decode steps
(expert ids compared), and the batched long-context decode for one sequence
of the 16 at 32768 cached positions.  Where the oracle cannot follow (the
8B model's whole 2048-token prompt), properties that hold at any size are
checked on the GPU: chunked prefill followed by decode equals a fresh
prefill of the same tokens, and kv_reset makes a run repeatable bit for bit.
"""
import gc

import numpy as np
import pytest

import oracle
from synth.weights import host_kv, host_weights, prompt
from synth.workloads import C135M, C8B, LONGCTX, MOE
from tests.gpu_util import MARGIN, assert_parity, compare_logits, decode, log, make_decoder, run_prefill

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def w8b():
    W = host_weights(C8B)
    yield W
    del W
    gc.collect()


def teacher_forced(dec, m, start_logits, pos, steps, what, moe_shape=None, cones=None):
    last = start_logits
    for i in range(steps):
        t = oracle.argmax(last)
        want = m.forward([t], pos + i, routes=moe_shape is not None, probs=moe_shape is not None)
        lg, am = decode(dec, [0], [t])
        st = compare_logits(lg[0], want["logits"], f"{what} decode {i}")
        log(what, "decode", i, st)
        n_cones = len(cones or [])
        if moe_shape is not None:
            cones = check_routes(dec, moe_shape, want, 1, f"{what} decode {i}", cones=cones, pos0=pos + i)
        if moe_shape is not None and any(p0 == pos + i for _, p0 in cones[n_cones:]):
            log(what, "decode", i, "this token's expert path flipped at a near-tie: logits not compared")
        else:
            assert_parity(st, f"{what} decode {i}")
        last = want["logits"]
    return last


def route_mismatch_ok(got, ref, probs, k, tie=1e-3):
    """End to end, the router sees the GPU's own normed input, which differs
    from the oracle's by the model's accumulated rounding (about 1e-4 to 1e-3
    relative in deep layers).  The chosen experts must match except where the
    oracle's k-th and (k+1)-th probabilities are closer than that (a near-tie,
    logged).  Their order in the top-k list does not enter the result (the
    routed experts are summed with their own weights), so sets are compared.
    Bit-exact ids on identical router inputs are checked separately
    (test_gpu_parity)."""
    p = np.sort(probs)[::-1]
    gap = (p[k - 1] - p[k]) / p[k - 1]
    return gap < tie, f"k-th gap {gap:.2e}"


def check_routes(dec, shape, want, rows, what, cones=None, pos0=0):
    """Expert sets of every (layer, token) against the oracle.  A set that
    differs at a near-tie (k-th gap < 1e-3) is a flip: that token then follows
    another, equally valid expert path (its own later layers are not
    compared), and its changed K/V reach every later token through attention,
    so inside the causal cone of a flip (later layers, later positions) only
    near-ties up to 1e-2 are accepted.
    Outside every cone the sets must match.  Returns the cones (layer,
    position) so later calls (decode steps) can continue the bookkeeping."""
    got = torch.empty((shape.n_layers, rows, shape.top_k), dtype=torch.int32, device="cuda")
    dec.debug_read_routes(got, rows)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    ref = want["routes"]
    cones = [] if cones is None else cones
    n_bad = 0
    for l in range(shape.n_layers):
        for i in range(rows):
            if set(got[l, i]) == set(ref[l, i]):
                continue
            if any(l > l0 and pos0 + i == p0 for l0, p0 in cones):
                continue    # the flipped token itself: another expert path, not comparable
            n_bad += 1
            inside = any(l > l0 and pos0 + i > p0 for l0, p0 in cones)
            p = np.sort(want["probs"][l, i])[::-1]
            gap = (p[shape.top_k - 1] - p[shape.top_k]) / p[shape.top_k - 1]
            log(what, f"route flip layer {l} pos {pos0 + i}: gpu {sorted(map(int, got[l, i]))} oracle {sorted(map(int, ref[l, i]))} "
                      f"k-th gap {gap:.2e}{' (inside an earlier cone)' if inside else ''}")
            assert gap < (1e-2 if inside else 1e-3), f"{what}: expert ids differ at layer {l} pos {pos0 + i}"
            cones.append((l, pos0 + i))
    log(what, "routes: flips", n_bad, "of", shape.n_layers * rows)
    return cones


def test_135m_full_prompt_and_decode():
    shape = C135M
    W = host_weights(shape)
    ids = prompt(shape, 512)
    m = oracle.Model(shape, W)
    want = m.prefill(ids, 128)["logits"]
    dec, _ = make_decoder(shape, W)
    got = run_prefill(dec, ids, 128)
    st = compare_logits(got, want, "135m prefill")
    log("135m prefill", st)
    assert_parity(st, "135m prefill")
    last = teacher_forced(dec, m, want, 512, 24, "135m")
    # then graph-replayed greedy decode (decode_run) at full size: each
    # token equals the oracle's wherever its top-2 margin exceeds 5e-2
    t = oracle.argmax(last)
    want = m.forward([t], 536)["logits"]
    lg, am = decode(dec, [0], [t])
    assert_parity(compare_logits(lg[0], want, "135m decode 24"), "135m decode 24")
    n = 12
    toks = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    dec.decode_run(0, n, toks)
    torch.cuda.synchronize()
    got = [int(x) for x in toks.cpu().numpy()]
    inputs = [int(am[0])] + got[:-1]
    clear = 0
    for i in range(n):
        w = m.forward([inputs[i]], 537 + i)["logits"]
        top2 = np.sort(w)[-2:]
        if top2[1] - top2[0] > MARGIN:
            assert got[i] == oracle.argmax(w), f"135m decode_run step {i}"
            clear += 1
    log("135m decode_run tokens", got, "checked against the oracle:", clear)
    assert clear >= 1


def test_8b_chunk_and_decode(w8b):
    shape = C8B.with_(max_seq=256)
    m = oracle.Model(shape, w8b)
    ids = prompt(shape, 128)
    want = m.forward(ids, 0)["logits"]
    dec, dw = make_decoder(shape, w8b)
    got = run_prefill(dec, ids, 128)
    st = compare_logits(got, want, "8b prefill")
    log("8b prefill", st)
    assert_parity(st, "8b prefill")
    teacher_forced(dec, m, want, 128, 3, "8b")
    dec.close()
    del dec, dw
    torch.cuda.empty_cache()


def test_8b_full_prompt_properties(w8b):
    """2048-token prompt in chunks of 128: decode after the chunked prefill
    equals a fresh one-chunk-longer recompute, and a reset run is bit-identical."""
    from synth.device import upload_weights
    from decoder_only_transformer_step_amd import Decoder
    shape = C8B.with_(max_seq=2304)
    dw = upload_weights(w8b)
    dec = Decoder(shape, dw)
    ids = [int(t) for t in prompt(shape, 2048)]
    a = run_prefill(dec, ids, 128)
    lg, am = decode(dec, [0], [ids[7]])
    assert np.all(np.isfinite(lg))
    dec.kv_reset(0)
    b = run_prefill(dec, ids, 128)
    assert np.array_equal(a, b)
    # the same 2049 tokens with chunk boundaries shifted by one, so token 2048
    # is the last row of a 128-row prefill chunk instead of a decode step
    dec.kv_reset(0)
    run_prefill(dec, ids[:1], 1)
    c = run_prefill(dec, ids[1:] + [ids[7]], 128, start=1)
    st = compare_logits(lg[0], c, "8b decode vs prefill")
    log("8b decode vs prefill", st)
    assert st["max_abs"] < 2e-2 and st["rel_l2"] < 1e-2
    dec.close()
    del dec, dw
    torch.cuda.empty_cache()


def test_moe_chunk_decode_and_routes():
    shape = MOE.with_(max_seq=256)
    W = host_weights(shape)
    m = oracle.Model(shape, W)
    ids = prompt(shape, 128)
    want = m.forward(ids, 0, routes=True, probs=True)
    dec, dw = make_decoder(shape, W)
    got = run_prefill(dec, ids, 128)
    st = compare_logits(got, want["logits"], "moe prefill")
    log("moe prefill", st)
    cones = check_routes(dec, shape, want, 128, "moe prefill")
    if any(p0 == 127 for _, p0 in cones):
        log("moe prefill: the last token's expert path flipped at a near-tie: logits not compared")
    else:
        assert_parity(st, "moe prefill")
    teacher_forced(dec, m, want["logits"], 128, 4, "moe", moe_shape=shape, cones=cones)
    dec.close()
    del dec, dw, W, m
    gc.collect()
    torch.cuda.empty_cache()


def test_longctx_batched_decode_one_sequence(w8b):
    from synth.device import device_kv, to_device, upload_weights
    from decoder_only_transformer_step_amd import Decoder
    shape = LONGCTX
    ctx = 32768
    dw = upload_weights(w8b)
    dec = Decoder(shape, dw)
    buf = None
    for s in range(1, shape.max_batch):
        for l in range(shape.n_layers):
            buf = device_kv(shape, s, l, ctx, out=buf)
            dec.kv_load(s, l, buf[0], buf[1], ctx)
    del buf
    m = oracle.Model(shape.with_(max_batch=1), w8b, max_seq=ctx + 4)
    for l in range(shape.n_layers):
        K, V = host_kv(shape, 0, l, ctx)
        m.kv_load(0, l, K, V, ctx)
        dec.kv_load(0, l, to_device(K), to_device(V), ctx)
        del K, V
    torch.cuda.synchronize()
    assert dec.seq_len(0) == ctx and dec.seq_len(15) == ctx
    toks = [int(t) for t in prompt(shape, shape.max_batch, seq=99)]
    seqs = list(range(shape.max_batch))
    for step in range(2):
        want = m.forward([toks[0]], ctx + step)["logits"]
        lg, am = decode(dec, seqs, toks)
        st = compare_logits(lg[0], want, f"longctx step {step}")
        log("longctx", step, st)
        assert_parity(st, f"longctx step {step}")
        assert np.all(np.isfinite(lg))
        toks = [int(a) for a in am]
        toks[0] = oracle.argmax(want)
    dec.close()
    del dec, dw, m
    gc.collect()
    torch.cuda.empty_cache()
