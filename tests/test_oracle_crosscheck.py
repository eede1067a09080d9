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


@pytest.mark.parametrize("variant", ["window", "softcap", "sinks", "qk_norm", "all"])
def test_attention_variants_match_numpy(variant):
    """Each attention variant (engine.zig Engine.forward: window and logit
    soft-cap handed to the attention, applyHeadNorm before RoPE; decoder.rs
    AttnWeights::sinks) in the C oracle against the vectorised numpy forward."""
    kw = {}
    if variant in ("window", "all"):
        kw["sliding_window"] = 3
    if variant in ("softcap", "all"):
        kw["attn_softcap"] = 0.7
    if variant in ("sinks", "all"):
        kw["attn_sinks"] = True
    if variant in ("qk_norm", "all"):
        kw["qk_norm"] = True
    s = small_shape(n_heads=4, n_kv_heads=2, qkv_bias=True, **kw)
    W = rand_weights(s)
    for L in W["layers"]:
        if s.attn_sinks:
            L["attn_sinks"] = np.random.default_rng(5).normal(size=s.n_heads).astype(np.float32)
        if s.qk_norm:
            g = np.random.default_rng(6)
            L["q_norm"] = (1 + 0.3 * g.normal(size=s.head_dim)).astype(np.float32)
            L["k_norm"] = (1 + 0.3 * g.normal(size=s.head_dim)).astype(np.float32)
    ids = synth.tokens(11, 23, s.vocab)
    got = oracle.Model(s, W).forward(ids, 0, logits_mode=2)["logits"]
    want = npref.forward(s, W, ids)
    assert np.abs(got - want).max() <= 1e-10 * np.abs(want).max()
    W_plain = dict(W, layers=[{k: v for k, v in L.items() if k != "attn_sinks"} for L in W["layers"]])
    plain = npref.forward(small_shape(n_heads=4, n_kv_heads=2, qkv_bias=True), W_plain, ids)
    assert np.abs(plain - want).max() > 1e-6 * np.abs(want).max()
