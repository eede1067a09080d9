"""Multi-position verify against the oracle.

Speculative decoding checks drafted tokens by running their positions
through the model in one pass that streams each weight matrix once, then
drops the KV rows of the drafts it rejects (pipeline.rs
Pipeline::generate_from_ids, forward_pair; truncate_last).  Here that pass
is prefill_chunk with every row's logits (logits_mode 2), and the rollback
is kv_truncate.  Each row's logits must meet the acceptance rule against the
oracle's, the kernel's greedy id of each row must be the lowest-index
maximum of its own logits, and a decode after a rollback must match the
oracle's decode after the same rollback.
"""
import numpy as np
import pytest

import oracle
from synth.weights import host_weights, prompt
from synth.workloads import C8B, TINY
from tests.gpu_util import assert_parity, compare_logits, decode, log, make_decoder, run_prefill

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SHAPES = {
    "tiny": (TINY, 16),
    # 8B-class layer shapes in two layers with a small vocabulary
    "8b2": (C8B.with_(name="gqa-8b-layers-2", n_layers=2, vocab=1024, max_seq=256), 40),
    # int8 weights: the verify pass streams the codes (the oracle runs on the
    # dequantised weights)
    "8b2-q8": (C8B.with_(name="gqa-8b-layers-2-q8", n_layers=2, vocab=1024, max_seq=256, weight_quant=1), 40),
}


@pytest.fixture(scope="module")
def models():
    cache = {}

    def get(which):
        if which not in cache:
            shape, P = SHAPES[which]
            cache[which] = (shape, P, host_weights(shape))
        return cache[which]
    return get


@pytest.mark.parametrize("n", [2, 4, 8])
@pytest.mark.parametrize("which", ["tiny", "8b2", "8b2-q8"])
def test_verify_rows_match_oracle(models, which, n):
    shape, P, W = models(which)
    ids = [int(t) for t in prompt(shape, P + n)]
    m = oracle.Model(shape, W)
    m.forward(ids[:P], 0, logits_mode=0)
    want = m.forward(ids[P:], P, logits_mode=2)["logits"]
    dec, _ = make_decoder(shape, W)
    run_prefill(dec, ids[:P], 128)
    logits = torch.full((n, shape.vocab), float("nan"), dtype=torch.float32, device="cuda")
    am = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    dec.prefill_chunk(0, ids[P:], P, logits_mode=2, logits=logits, argmax=am)
    torch.cuda.synchronize()
    got, gam = logits.cpu().numpy(), am.cpu().numpy()
    assert dec.seq_len(0) == P + n
    for i in range(n):
        st = compare_logits(got[i], want[i], f"{which} verify {n} row {i}")
        log(which, "verify", n, "row", i, st)
        assert_parity(st, f"{which} verify {n} row {i}")
        assert gam[i] == int(np.argmax(got[i])), (i, gam[i])
    dec.close()


@pytest.mark.parametrize("keep", [0, 1, 3])
@pytest.mark.parametrize("which", ["tiny", "8b2"])
def test_rollback_then_decode_matches_oracle(models, which, keep):
    """Verify four drafts, keep the first `keep`, decode the next token."""
    shape, P, W = models(which)
    n = 4
    ids = [int(t) for t in prompt(shape, P + n + 1)]
    nxt = ids[P + n]
    m = oracle.Model(shape, W)
    m.forward(ids[:P], 0, logits_mode=0)
    m.forward(ids[P:P + n], P, logits_mode=0)
    m.truncate(0, P + keep)
    want = m.forward([nxt], P + keep)["logits"]
    dec, _ = make_decoder(shape, W)
    run_prefill(dec, ids[:P], 128)
    dec.prefill_chunk(0, ids[P:P + n], P, logits_mode=2)
    dec.kv_truncate(0, P + keep)
    assert dec.seq_len(0) == P + keep
    with pytest.raises(Exception):
        dec.decode_step([0], None)      # the rolled-back sequence has no greedy token to feed back
    with pytest.raises(Exception):
        dec.kv_truncate(0, P + keep + 1)
    lg, am = decode(dec, [0], [nxt])
    st = compare_logits(lg[0], want, f"{which} keep {keep}")
    log(which, "rollback keep", keep, st)
    assert_parity(st, f"{which} rollback keep {keep}")
    assert dec.seq_len(0) == P + keep + 1
    dec.close()


@pytest.mark.parametrize("which", ["tiny", "8b2"])
def test_accepted_verify_feeds_its_last_greedy_token(models, which):
    """After a verify whose drafts are all accepted (no rollback), a decode
    with tokens = NULL feeds the greedy token of the verify's LAST row, the
    one after the last drafted position: every row of the pass computes a
    greedy id, and only the last row's may become the sequence's next
    token.  The logits equal those of a decode given that token."""
    shape, P, W = models(which)
    n = 4
    ids = [int(t) for t in prompt(shape, P + n)]
    dec, _ = make_decoder(shape, W)
    run_prefill(dec, ids[:P], 128)
    am = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    dec.prefill_chunk(0, ids[P:], P, logits_mode=2, argmax=am)
    torch.cuda.synchronize()
    last = int(am.cpu().numpy()[-1])
    lg_fed, _ = decode(dec, [0], None)
    dec.kv_truncate(0, P + n)
    lg_given, _ = decode(dec, [0], [last])
    assert np.array_equal(lg_fed, lg_given), which
    dec.close()
