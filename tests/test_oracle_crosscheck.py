"""The C oracle against an independent vectorised numpy forward (tests/npref.py)
on the tiny workload and on small MoE / biased / tied shapes."""
import numpy as np
import pytest

import oracle
import synth
from synth.weights import host_weights, prompt
from synth.workloads import TINY
from tests import npref
from tests.test_oracle_pins import moe_shape, rand_weights, small_shape


def test_tiny_workload_prefill_then_decode_matches_numpy():
    W = host_weights(TINY)
    ids = list(prompt(TINY, 16))
    m = oracle.Model(TINY, W, kv_bf16=False)     # numpy reference keeps an exact cache
    logits = [m.forward(ids, 0)["logits"]]
    for i in range(8):                           # greedy continuation
        nxt = oracle.argmax(logits[-1])
        ids.append(nxt)
        logits.append(m.forward([nxt], 16 + i)["logits"])
    ref = npref.forward(TINY, W, ids)
    got = np.stack(logits)
    want = ref[15:]
    assert np.abs(got - want).max() <= 1e-10 * np.abs(want).max()


@pytest.mark.parametrize("kind", ["moe", "moe_renorm", "tied_bias"])
def test_small_shapes_match_numpy(kind):
    if kind == "moe":
        s = moe_shape(n_experts=6, top_k=2, shared_inter=16, shared_gate=True, qkv_bias=True, n_layers=2)
    elif kind == "moe_renorm":
        s = moe_shape(n_experts=5, top_k=3, norm_topk_prob=1, n_layers=2)
    else:
        s = small_shape(tied=True, qkv_bias=True, n_heads=6, n_kv_heads=2)
    W = rand_weights(s)
    ids = synth.tokens(11, 17, s.vocab)
    got = oracle.Model(s, W).forward(ids, 0, logits_mode=2)["logits"]
    want = npref.forward(s, W, ids)
    assert np.abs(got - want).max() <= 1e-10 * np.abs(want).max()
