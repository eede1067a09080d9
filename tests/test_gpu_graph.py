"""decode_run: greedy decode steps replayed from one captured HIP graph.

The captured step reads its position from device memory and is replayed
once per token; between two runs the program does its own eager step.  Each
generated token must be the oracle's greedy token wherever the oracle's
top-2 margin exceeds 5e-2 (the oracle is fed the tokens the GPU produced),
the last logits must meet the acceptance rule, and the eager decoder on the
same inputs must agree with the graph-replayed one on those tokens.
"""
import numpy as np
import pytest

import oracle
from synth.weights import host_weights, prompt
from synth.workloads import C8B, TINY
from tests.gpu_util import MARGIN, assert_parity, compare_logits, decode, log, make_decoder, run_prefill

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def shapes():
    from tests.test_gpu_parity import small_moe
    return {
        "tiny": (TINY, 16, 16),
        "8b2": (C8B.with_(name="gqa-8b-layers-2", n_layers=2, vocab=1024, max_seq=512), 130, 128),
        "moe": (small_moe(), 24, 32),
        "moe-q8": (small_moe().with_(name="moe-small-q8", weight_quant=1), 24, 32),
        # every option at once, the run crossing a page boundary (positions
        # 120..131 over 32-position pages) with keys outside the window
        "8b2-all": (C8B.with_(name="gqa-8b-layers-2-all", n_layers=2, vocab=1024, max_seq=512, weight_quant=1,
                              sliding_window=100, attn_softcap=2.0, attn_sinks=True, qk_norm=True,
                              kv_page_size=32, kv_pages=8), 120, 64),
    }


@pytest.mark.parametrize("which", ["tiny", "8b2", "moe", "moe-q8", "8b2-all"])
def test_decode_run_matches_oracle_and_eager(which):
    shape, P, chunk = shapes()[which]
    W = host_weights(shape)
    ids = prompt(shape, P)
    dec, _ = make_decoder(shape, W)
    g0 = int(np.argmax(run_prefill(dec, ids, chunk)))   # the prefill's greedy token: step 0's input
    n1, n2 = 6, 5
    t1 = torch.full((n1,), -1, dtype=torch.int32, device="cuda")
    dec.decode_run(0, n1, t1)
    # an eager step between the two runs (feeds back the last greedy token)
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    mid_logits = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
    dec.decode_step([0], None, logits=mid_logits, argmax=am)
    t2 = torch.full((n2,), -1, dtype=torch.int32, device="cuda")
    dec.decode_run(0, n2, t2)
    torch.cuda.synchronize()
    assert dec.seq_len(0) == P + n1 + 1 + n2
    got = [int(t) for t in t1.cpu().numpy()] + [int(am.cpu().numpy()[0])] + [int(t) for t in t2.cpu().numpy()]
    inputs = [g0] + got[:-1]

    # the oracle, fed the tokens the GPU generated: step i reads inputs[i] at
    # position P + i and must emit got[i] wherever its margin is clear
    m = oracle.Model(shape, W)
    m.prefill(ids, chunk)
    wants = []
    for i, t in enumerate(got):
        want = m.forward([inputs[i]], P + i)["logits"]
        wants.append(want)
        top2 = np.sort(want)[-2:]
        if top2[1] - top2[0] > MARGIN:
            assert t == oracle.argmax(want), f"{which} step {i}: {t} vs {oracle.argmax(want)}"
        if i == n1:   # the eager step's logits
            assert_parity(compare_logits(mid_logits.cpu().numpy()[0], want, f"{which} eager step"), which)
    clear = sum(1 for w in wants if np.diff(np.sort(w)[-2:])[0] > MARGIN)
    log(which, "decode_run tokens", got, "checked against the oracle:", clear)
    assert clear >= 1

    # an eager decoder fed the same tokens (contiguous cache) agrees where
    # the margin is clear
    eager, _ = make_decoder(shape.with_(kv_page_size=0, kv_pages=0), W)
    run_prefill(eager, ids, chunk)
    for i in range(len(got)):
        _, ia = decode(eager, [0], [inputs[i]])
        top2 = np.sort(wants[i])[-2:]
        if top2[1] - top2[0] > MARGIN:
            assert int(ia[0]) == got[i], f"{which} eager step {i}"
    dec.close()
    eager.close()


def test_decode_run_refusals_change_nothing():
    """Calls decode_run must refuse: no previous greedy token (after a
    rollback), a run past max_seq, node timers on, n_steps < 1.  Each is
    refused before anything runs; the sequence then still decodes as an
    untouched one would."""
    from decoder_only_transformer_step_amd.binding import DecoderError
    shape = TINY
    W = host_weights(shape)
    ids = prompt(shape, 16)
    dec, _ = make_decoder(shape, W)
    ref, _ = make_decoder(shape, W)
    for d in (dec, ref):
        run_prefill(d, ids, 16)
    toks = torch.zeros(shape.max_seq, dtype=torch.int32, device="cuda")
    with pytest.raises(DecoderError):
        dec.decode_run(0, shape.max_seq - 16 + 1, toks)      # past max_seq
    with pytest.raises(DecoderError):
        dec.decode_run(0, 0, toks)
    dec.stats_enable()
    with pytest.raises(DecoderError):
        dec.decode_run(0, 2, toks)
    dec.stats_enable(())
    assert dec.seq_len(0) == 16
    a = decode(dec, [0], None)
    b = decode(ref, [0], None)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    dec.kv_truncate(0, 17)                                   # forgets the greedy token
    with pytest.raises(DecoderError):
        dec.decode_run(0, 2, toks)
    # a run that ends exactly at max_seq is accepted
    dec.kv_truncate(0, 16)
    decode(dec, [0], [int(ids[-1])])
    n = shape.max_seq - dec.seq_len(0)
    dec.decode_run(0, n, toks)
    assert dec.seq_len(0) == shape.max_seq
    dec.close()
    ref.close()


def test_decode_run_on_a_caller_stream():
    """A decoder on a caller's (non-default) stream: the prefill is only
    enqueued there when decode_run starts, so the run must order itself
    after it.  Tokens equal those of the same run on the default stream."""
    from decoder_only_transformer_step_amd import Decoder
    from synth.device import upload_weights
    shape, P, chunk = shapes()["8b2"]
    W = host_weights(shape)
    ids = [int(t) for t in prompt(shape, P)]
    dw = upload_weights(W)
    torch.cuda.synchronize()                # the uploads ran on the default stream
    out = []
    for stream in (torch.cuda.Stream(), None):
        dec = Decoder(shape, dw, stream=stream)
        torch.cuda.synchronize()
        logits = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
        for c0 in range(0, P, chunk):
            part = ids[c0:c0 + chunk]
            dec.prefill_chunk(0, part, c0, logits_mode=1, logits=logits)
        toks = torch.full((8,), -1, dtype=torch.int32, device="cuda")
        dec.decode_run(0, 8, toks)          # no host synchronisation before it
        torch.cuda.synchronize()
        out.append([int(t) for t in toks.cpu().numpy()])
        dec.close()
    log("caller-stream decode_run", out[0], "default stream", out[1])
    assert out[0] == out[1]
