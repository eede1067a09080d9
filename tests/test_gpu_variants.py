"""Attention variants against the oracle: a sliding window, a logit soft-cap,
per-head sink logits and per-head QK-norm (engine.zig Engine.forward hands
its attention a soft-cap and, on a sliding layer, a window, and
applyHeadNorm norms q and k heads before RoPE; decoder.rs AttnWeights::sinks),
alone and together.  Each runs a chunked prefill (several rows per block
and several key splits on the 8B shape, with the window crossing chunk and
split boundaries) and teacher-forced decode steps, logits compared with the
acceptance rule.
"""
import pytest

import oracle
from synth.weights import host_weights, prompt
from synth.workloads import C8B, TINY
from tests.gpu_util import assert_parity, compare_logits, decode, log, make_decoder, run_prefill

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# (base shape, prompt length, chunk, decode steps, window, soft-cap).  The
# caps sit near the typical scaled score of each shape (about 0.1 for the
# tiny model, about 1.6 for the 8B shape), so tanh is far from linear.
BASES = {
    "tiny": (TINY, 16, 16, 8, 8, 0.05),
    "8b2": (C8B.with_(name="gqa-8b-layers-2", n_layers=2, vocab=1024, max_seq=512), 200, 128, 6, 100, 2.0),
}
VARIANTS = ("window", "softcap", "sinks", "qknorm", "all")


def variant_shape(which, variant):
    base, _, _, _, W, cap = BASES[which]
    kw = {}
    if variant in ("window", "all"):
        kw["sliding_window"] = W
    if variant in ("softcap", "all"):
        kw["attn_softcap"] = cap
    if variant in ("sinks", "all"):
        kw["attn_sinks"] = True
    if variant in ("qknorm", "all"):
        kw["qk_norm"] = True
    return base.with_(name=f"{base.name}-{variant}", **kw)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("which", ["tiny", "8b2"])
def test_variant_prefill_and_decode(which, variant):
    _, P, chunk, steps, _, _ = BASES[which]
    shape = variant_shape(which, variant)
    W = host_weights(shape)
    ids = prompt(shape, P)
    m = oracle.Model(shape, W)
    want = m.prefill(ids, chunk)["logits"]
    dec, _ = make_decoder(shape, W)
    got = run_prefill(dec, ids, chunk)
    st = compare_logits(got, want, f"{which} {variant} prefill")
    log(which, variant, "prefill", st)
    assert_parity(st, f"{which} {variant} prefill")
    for i in range(steps):
        t = oracle.argmax(want)
        want = m.forward([t], P + i)["logits"]
        lg, _ = decode(dec, [0], [t])
        st = compare_logits(lg[0], want, f"{which} {variant} decode {i}")
        log(which, variant, "decode", i, st)
        assert_parity(st, f"{which} {variant} decode {i}")
    dec.close()


def test_variants_change_the_result():
    """Each variant moves the oracle's logits (so the parity tests above
    exercise it), and a window covering every position changes nothing."""
    _, P, chunk, _, _, _ = BASES["tiny"]
    plain_shape = TINY
    W = host_weights(plain_shape)
    ids = prompt(plain_shape, P)
    plain = oracle.Model(plain_shape, W).prefill(ids, chunk)["logits"]
    for variant in VARIANTS:
        s = variant_shape("tiny", variant)
        got = oracle.Model(s, host_weights(s)).prefill(ids, chunk)["logits"]
        assert abs(got - plain).max() > 1e-3, variant
    wide = TINY.with_(sliding_window=TINY.max_seq)
    assert (oracle.Model(wide, W).prefill(ids, chunk)["logits"] == plain).all()
