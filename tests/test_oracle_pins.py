"""Pins of the fp64 oracle to facts other than itself.

Each test checks the oracle against a closed form, an invariant, a special
case that reduces to a textbook routine, or brute force on tiny inputs.  The
cases are chosen so that a plausible slip (a dropped term, a wrong sign or
index, a transposed operand) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from synth.weights import host_weights, prompt
from synth.workloads import TINY, Shape

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(0)


def bits(x):
    """bf16 bit patterns of values that are exactly representable in bf16."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def rand_bits(shape, sigma=0.5):
    n = int(np.prod(shape))
    return synth.normal_bf16(n, int(rng.integers(1, 2**62)), sigma).reshape(shape)


def widen(b):
    return synth.bf16_to_f32(b).astype(np.float64)


# ---------------------------------------------------------------- RMSNorm --

def test_rmsnorm_unit_rms_before_gain():
    x = rng.normal(size=777) * 3.7
    eps = 1e-5
    a = oracle.rmsnorm(x, np.ones(777), eps)
    ms = np.mean(x * x)
    assert math.isclose(np.sqrt(np.mean(a * a)), np.sqrt(ms / (ms + eps)), rel_tol=1e-13)


def test_rmsnorm_constant_vector_closed_form():
    for c in (0.5, 2.0, 1e-3):
        a = oracle.rmsnorm(np.full(64, c), np.ones(64), 1e-5)
        assert np.allclose(a, c / math.sqrt(c * c + 1e-5), rtol=1e-14, atol=0)


def test_rmsnorm_gain_is_elementwise_after_normalisation():
    x = rng.normal(size=32)
    g = rng.normal(size=32).astype(np.float32)
    a1 = oracle.rmsnorm(x, np.ones(32), 1e-6)
    ag = oracle.rmsnorm(x, g, 1e-6)
    assert np.allclose(ag, a1 * g.astype(np.float64), rtol=1e-14, atol=1e-15)


# ------------------------------------------------------------------- RoPE --

@pytest.mark.parametrize("d,base", [(64, 1e4), (128, 5e5), (8, 10.0)])
def test_rope_single_pair_closed_form(d, base):
    # Unit vector on element i rotates into element i + d/2 by pos * base^(-2i/d).
    for i in (0, 1, d // 2 - 1):
        for pos in (1, 7, 2047):
            v = np.zeros(d)
            v[i] = 1.0
            r = oracle.rope(v, 1, d, pos, base)
            ang = pos * base ** (-2.0 * i / d)
            want = np.zeros(d)
            want[i] = math.cos(ang)
            want[i + d // 2] = math.sin(ang)
            assert np.allclose(r, want, atol=1e-12)
            # and the partner rotates the other way round
            v = np.zeros(d)
            v[i + d // 2] = 1.0
            r = oracle.rope(v, 1, d, pos, base)
            want = np.zeros(d)
            want[i] = -math.sin(ang)
            want[i + d // 2] = math.cos(ang)
            assert np.allclose(r, want, atol=1e-12)


def test_rope_identity_at_zero_and_norm_preserving():
    v = rng.normal(size=4 * 64)
    assert np.array_equal(oracle.rope(v, 4, 64, 0, 1e4), v)
    r = oracle.rope(v, 4, 64, 12345, 1e4)
    for h in range(4):
        a, b = v[h * 64:(h + 1) * 64], r[h * 64:(h + 1) * 64]
        assert math.isclose(np.linalg.norm(a), np.linalg.norm(b), rel_tol=1e-13)
        pa = a[:32] ** 2 + a[32:] ** 2
        pb = b[:32] ** 2 + b[32:] ** 2
        assert np.allclose(pa, pb, rtol=1e-12)


def test_rope_relative_position():
    # <R_m q, R_n k> depends only on m - n.
    d = 64
    q, k = rng.normal(size=d), rng.normal(size=d)
    for m, n in ((10, 3), (500, 100), (7, 7)):
        lhs = oracle.rope(q, 1, d, m, 1e4) @ oracle.rope(k, 1, d, n, 1e4)
        rhs = oracle.rope(q, 1, d, m - n, 1e4) @ k
        assert math.isclose(lhs, rhs, rel_tol=1e-10, abs_tol=1e-11)


# -------------------------------------------------------------- attention --

def test_attention_single_key_returns_v():
    Hq, Hkv, d = 4, 2, 16
    q = rng.normal(size=Hq * d)
    k = rng.normal(size=(1, Hkv * d))
    v = rng.normal(size=(1, Hkv * d))
    o = oracle.attend(q, k, v, Hq, Hkv, d).reshape(Hq, d)
    for h in range(Hq):
        g = h * Hkv // Hq
        assert np.allclose(o[h], v[0, g * d:(g + 1) * d], rtol=0, atol=1e-15)


def test_attention_identical_keys_give_mean_of_v():
    Hq, Hkv, d, T = 2, 1, 8, 9
    q = rng.normal(size=Hq * d)
    k = np.tile(rng.normal(size=(1, d)), (T, 1))
    v = rng.normal(size=(T, d))
    o = oracle.attend(q, k, v, Hq, Hkv, d).reshape(Hq, d)
    assert np.allclose(o, v.mean(axis=0), atol=1e-14)


def test_attention_dominant_score_selects_its_value():
    d, T = 8, 5
    q = np.zeros(d)
    q[0] = 1.0
    k = np.zeros((T, d))
    k[3, 0] = 1e4                          # score 1e4/sqrt(8) dominates
    v = rng.normal(size=(T, d))
    o = oracle.attend(q, k, v, 1, 1, d)
    assert np.allclose(o, v[3], atol=1e-12)


def test_attention_softmax_weights_closed_form():
    # two keys: weights are the logistic of the scaled score difference
    d = 4
    q = np.array([1.0, 0, 0, 0])
    k = np.array([[0.0, 0, 0, 0], [3.0, 0, 0, 0]])
    v = np.array([[1.0, 0, 0, 0], [0.0, 1, 0, 0]])
    o = oracle.attend(q, k, v, 1, 1, d)
    w1 = 1.0 / (1.0 + math.exp(-3.0 / 2.0))
    assert np.allclose(o, [1 - w1, w1, 0, 0], atol=1e-15)


# attention variants (engine.zig Engine.forward: logit soft-cap and sliding
# window handed to the attention; decoder.rs AttnWeights::sinks)

def test_window_keeps_exactly_the_most_recent_keys():
    Hq, Hkv, d, T = 4, 2, 16, 13
    q = rng.normal(size=Hq * d)
    k = rng.normal(size=(T, Hkv * d))
    v = rng.normal(size=(T, Hkv * d))
    plain = oracle.attend(q, k, v, Hq, Hkv, d)
    for W in (T, T + 5):                   # a window covering every key changes nothing
        assert np.array_equal(oracle.attend(q, k, v, Hq, Hkv, d, window=W), plain)
    for W in (1, 4, T - 1):                # the plain attention over the last W rows
        got = oracle.attend(q, k, v, Hq, Hkv, d, window=W)
        assert np.array_equal(got, oracle.attend(q, k[T - W:], v[T - W:], Hq, Hkv, d))
        assert not np.allclose(got, plain)
    one = oracle.attend(q, k, v, Hq, Hkv, d, window=1).reshape(Hq, d)
    for h in range(Hq):                    # window 1: the query's own value
        g = h * Hkv // Hq
        assert np.array_equal(one[h], v[T - 1, g * d:(g + 1) * d])


def test_softcap_closed_form():
    # cap 1, raw scaled scores +-atanh(1/2): capped scores +-1/2, so the two
    # weights are the logistic of 1 and of -1
    d = 4
    a = math.atanh(0.5) * 2.0              # scaled by 1/sqrt(4) = 1/2 inside
    q = np.array([1.0, 0, 0, 0])
    k = np.array([[a, 0, 0, 0], [-a, 0, 0, 0]])
    v = np.array([[1.0, 0, 0, 0], [0.0, 1, 0, 0]])
    o = oracle.attend(q, k, v, 1, 1, d, softcap=1.0)
    assert np.allclose(o, [0.7310585786300049, 0.2689414213699951, 0, 0], rtol=0, atol=1e-15)
    # a cap far above every score leaves the plain softmax (tanh(x) = x - x^3/3 ...)
    Hq, Hkv, d, T = 2, 1, 8, 7
    q = rng.normal(size=Hq * d)
    k = rng.normal(size=(T, d))
    v = rng.normal(size=(T, d))
    assert np.allclose(oracle.attend(q, k, v, Hq, Hkv, d, softcap=1e6), oracle.attend(q, k, v, Hq, Hkv, d),
                       rtol=0, atol=1e-10)


def test_sinks_closed_form_and_reductions():
    Hq, Hkv, d, T = 2, 1, 8, 6
    v = rng.normal(size=(T, d))
    # zero query: every score is 0, so with a sink logit of 0 the keys share
    # T/(T+1) of the weight: the output is T/(T+1) times the mean of V
    o = oracle.attend(np.zeros(Hq * d), rng.normal(size=(T, d)), v, Hq, Hkv, d,
                      sinks=np.zeros(Hq, np.float32)).reshape(Hq, d)
    assert np.allclose(o, v.mean(axis=0) * T / (T + 1), rtol=0, atol=1e-15)
    # a sink far below every score changes nothing; a sink far above takes all weight
    q = rng.normal(size=Hq * d)
    k = rng.normal(size=(T, d))
    plain = oracle.attend(q, k, v, Hq, Hkv, d)
    assert np.array_equal(oracle.attend(q, k, v, Hq, Hkv, d, sinks=np.full(Hq, -1e30, np.float32)), plain)
    assert np.allclose(oracle.attend(q, k, v, Hq, Hkv, d, sinks=np.full(Hq, 80.0, np.float32)), 0,
                       rtol=0, atol=1e-30)
    # one sink per head: head 1's sink leaves head 0 alone
    mixed = oracle.attend(q, k, v, Hq, Hkv, d, sinks=np.array([-1e30, 0.5], np.float32)).reshape(Hq, d)
    assert np.array_equal(mixed[0], plain.reshape(Hq, d)[0])
    assert not np.allclose(mixed[1], plain.reshape(Hq, d)[1])


def test_model_variants_reduce_to_the_plain_model():
    s = small_shape()
    W = rand_weights(s)
    ids = synth.tokens(12, 21, s.vocab)
    plain = oracle.Model(s, W).forward(ids, 0, logits_mode=2)["logits"]
    wide = oracle.Model(s.with_(sliding_window=s.max_seq), W).forward(ids, 0, logits_mode=2)["logits"]
    assert np.array_equal(wide, plain)
    Ws = dict(W, layers=[dict(L, attn_sinks=np.full(s.n_heads, -1e30, np.float32)) for L in W["layers"]])
    assert np.array_equal(oracle.Model(s, Ws).forward(ids, 0, logits_mode=2)["logits"], plain)
    narrow = oracle.Model(s.with_(sliding_window=4), W).forward(ids, 0, logits_mode=2)["logits"]
    assert np.array_equal(narrow[:4], plain[:4])       # positions 0..3 see every key anyway
    assert not np.allclose(narrow[4:], plain[4:])


def test_qk_norm_makes_each_head_scale_free():
    """With the per-head RMSNorm of q and k (engine.zig applyHeadNorm, before
    RoPE) and eps 0, scaling one q head's or one k head's weight rows by a
    power of two (exact in bf16) leaves the logits unchanged; without it they
    move.  A norm over the wrong slice (the whole q vector, or across heads)
    would not cancel a single head's scale."""
    for qk in (True, False):
        s = small_shape(qk_norm=qk, rms_eps=0.0)
        W = rand_weights(s)
        for L in W["layers"]:
            L["q_norm"] = (1 + 0.2 * rng.normal(size=s.head_dim)).astype(np.float32)
            L["k_norm"] = (1 + 0.2 * rng.normal(size=s.head_dim)).astype(np.float32)
        ids = synth.tokens(9, 31, s.vocab)
        base = oracle.Model(s, W).forward(ids, 0, logits_mode=2)["logits"]
        d, H = s.head_dim, s.hidden
        W2 = dict(W, layers=[dict(L) for L in W["layers"]])
        wq = widen(W2["layers"][0]["w_qkv"]).reshape(s.qkv_rows, H).copy()
        wq[1 * d:2 * d] *= 4.0                          # q head 1
        wq[s.q_dim + 0 * d:s.q_dim + 1 * d] *= 0.5      # k head 0
        W2["layers"][0]["w_qkv"] = bits(wq)
        got = oracle.Model(s, W2).forward(ids, 0, logits_mode=2)["logits"]
        if qk:
            assert np.allclose(got, base, rtol=0, atol=1e-12 * np.abs(base).max())
        else:
            assert not np.allclose(got, base, rtol=0, atol=1e-6)


def test_gqa_equals_mha_with_repeated_kv_heads():
    Hq, Hkv, d, T = 8, 2, 16, 11
    q = rng.normal(size=Hq * d)
    k = rng.normal(size=(T, Hkv, d))
    v = rng.normal(size=(T, Hkv, d))
    o_gqa = oracle.attend(q, k.reshape(T, -1), v.reshape(T, -1), Hq, Hkv, d)
    rep = Hq // Hkv                        # contiguous groups: q head h reads kv head h // rep
    k_rep = np.repeat(k, rep, axis=1)
    v_rep = np.repeat(v, rep, axis=1)
    o_mha = oracle.attend(q, k_rep.reshape(T, -1), v_rep.reshape(T, -1), Hq, Hq, d)
    assert np.array_equal(o_gqa, o_mha)
    # and the MHA case agrees with a brute-force per-head softmax
    qh = q.reshape(Hq, d)
    for h in range(Hq):
        s = k_rep[:, h, :] @ qh[h] / math.sqrt(d)
        p = np.exp(s - s.max())
        p /= p.sum()
        assert np.allclose(o_mha.reshape(Hq, d)[h], p @ v_rep[:, h, :], atol=1e-13)


# -------------------------------------------------------- linear and FFN --

@pytest.mark.parametrize("rows,cols,n", [(37, 53, 1), (64, 17, 6), (5, 300, 3)])
def test_matmul_matches_numpy(rows, cols, n):
    W = rand_bits((rows, cols))
    X = rng.normal(size=(n, cols))
    Y = oracle.matmul(W, rows, cols, X)
    ref = X @ widen(W).T
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-13)


def test_silu_values():
    assert oracle.silu(0.0) == 0.0
    assert math.isclose(oracle.silu(1.0), 1.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-15)
    assert math.isclose(oracle.silu(30.0), 30.0, rel_tol=1e-12)
    assert abs(oracle.silu(-40.0)) < 1e-15
    assert oracle.sigmoid(0.0) == 0.5


# ----------------------------------------------------------------- router --

def test_route_topk_and_ties():
    logits = np.array([0.1, 2.0, 2.0, -1.0, 0.5])
    idx, w, p = oracle.route(logits, 2, 0)
    assert list(idx) == [1, 2]                    # tie goes to the lower index first
    ref = np.exp(logits - logits.max())
    ref /= ref.sum()
    assert np.allclose(p, ref, rtol=1e-15)
    assert np.allclose(w, ref[[1, 2]], rtol=1e-15)
    idx, w, _ = oracle.route(logits, 3, 1)
    assert list(idx) == [1, 2, 4]
    assert math.isclose(w.sum(), 1.0, rel_tol=1e-15)
    idx, w, _ = oracle.route(np.zeros(6), 6, 0)
    assert list(idx) == list(range(6))
    assert np.allclose(w, 1 / 6, rtol=1e-15)


def test_argmax_lowest_index_on_ties():
    assert oracle.argmax([1.0, 3.0, 3.0, 2.0]) == 1
    assert oracle.argmax([-5.0]) == 0


# ------------------------------------------------------------ whole model --

def small_shape(**kw):
    # exact-arithmetic pins use an fp64 KV cache; the bf16 cache has its own test
    base = dict(name="pin", hidden=32, n_layers=2, n_heads=4, n_kv_heads=2, head_dim=8,
                vocab=64, ffn_inter=48, rope_base=1e4, rms_eps=1e-5, max_seq=32, max_chunk=16,
                kv_bf16=False)
    base.update(kw)
    return Shape(**base)


def rand_weights(shape, sigma=0.3):
    s = shape
    H = s.hidden
    W = {"embed": rand_bits((s.vocab, H), sigma), "final_norm": np.ones(H, np.float32)}
    W["lm_head"] = W["embed"] if s.tied else rand_bits((s.vocab, H), sigma)
    W["layers"] = []
    for _ in range(s.n_layers):
        L = {"attn_norm": (1 + 0.1 * rng.normal(size=H)).astype(np.float32),
             "ffn_norm": (1 + 0.1 * rng.normal(size=H)).astype(np.float32),
             "w_qkv": rand_bits((s.qkv_rows, H), sigma), "w_o": rand_bits((H, s.q_dim), sigma)}
        if s.qkv_bias:
            L["b_qkv"] = widen(rand_bits((s.qkv_rows,), sigma)).astype(np.float32)
        if s.is_moe:
            E, Ie, Is = s.n_experts, s.expert_inter, s.shared_inter
            L["w_router"] = rand_bits((E, H), 1.0)
            L["w_exp_gate_up"] = rand_bits((E, 2 * Ie, H), sigma)
            L["w_exp_down"] = rand_bits((E, H, Ie), sigma)
            if Is:
                L["w_sh_gate_up"] = rand_bits((2 * Is, H), sigma)
                L["w_sh_down"] = rand_bits((H, Is), sigma)
                if s.shared_gate:
                    L["w_sh_gate"] = rand_bits((H,), sigma)
        else:
            L["w_gate_up"] = rand_bits((2 * s.ffn_inter, H), sigma)
            L["w_down"] = rand_bits((H, s.ffn_inter), sigma)
        W["layers"].append(L)
    return W


def test_hand_case_closed_form():
    """One layer, one head: q = k = 0, v = o = I, no FFN, lm_head = I (golden fixture)."""
    with open(os.path.join(GOLDEN, "hand_case_h4.json")) as f:
        case = json.load(f)
    eps = case["rms_eps"]
    s = small_shape(hidden=4, n_layers=1, n_heads=1, n_kv_heads=1, head_dim=4, vocab=4,
                    ffn_inter=4, rms_eps=eps)
    I4 = np.eye(4, dtype=np.float32)
    embed = np.zeros((4, 4), np.float32)
    embed[0] = case["embed_row0"]
    W = {"embed": bits(embed), "lm_head": bits(I4), "final_norm": np.ones(4, np.float32),
         "layers": [{"attn_norm": np.ones(4, np.float32), "ffn_norm": np.ones(4, np.float32),
                     "w_qkv": bits(np.concatenate([np.zeros((8, 4), np.float32), I4])),
                     "w_o": bits(I4), "w_gate_up": bits(np.zeros((8, 4), np.float32)),
                     "w_down": bits(np.zeros((4, 4), np.float32))}]}
    m = oracle.Model(s, W)
    lg = m.forward([0], 0)["logits"]
    # a = x / sqrt(1 + eps); x1 = x + a; logits = x1 / sqrt(mean(x1^2) + eps)
    c = 2.0 + 2.0 / math.sqrt(1.0 + eps)
    want = np.array([c / math.sqrt(c * c / 4.0 + eps), 0, 0, 0])
    assert np.allclose(lg, want, rtol=1e-14, atol=0)
    assert np.allclose(lg, case["expected_logits"], rtol=1e-12, atol=0)


def test_bias_reaches_v_before_attention():
    # W_qkv = 0 with a bias: q = b_q, k = b_k rotated, v = b_v; one key, so the
    # attention output is b_v and x gains W_o b_v.
    s = small_shape(hidden=4, n_layers=1, n_heads=1, n_kv_heads=1, head_dim=4, vocab=4,
                    ffn_inter=4, qkv_bias=True)
    I4 = np.eye(4, dtype=np.float32)
    bias = np.zeros(12, np.float32)
    bias[8:12] = [0.5, -1.0, 0.25, 2.0]
    embed = np.zeros((4, 4), np.float32)
    embed[0] = [1.0, 0, 0, 0]
    W = {"embed": bits(embed), "lm_head": bits(I4), "final_norm": np.ones(4, np.float32),
         "layers": [{"attn_norm": np.ones(4, np.float32), "ffn_norm": np.ones(4, np.float32),
                     "w_qkv": bits(np.zeros((12, 4), np.float32)), "b_qkv": bias,
                     "w_o": bits(I4), "w_gate_up": bits(np.zeros((8, 4), np.float32)),
                     "w_down": bits(np.zeros((4, 4), np.float32))}]}
    out = oracle.Model(s, W).forward([0], 0, trace=True)
    x1 = out["trace"][1, 0]
    assert np.allclose(x1, [1.5, -1.0, 0.25, 2.0], atol=1e-15)


def _kv_load_model(w_q):
    """H = 4, one layer, two heads of d = 2 with one kv head each; W_k = W_v = 0
    (the query's own key and value are zero), W_o = I, no FFN, lm-head = I,
    E[0] = (1, 0, 0, 0)."""
    s = small_shape(hidden=4, n_layers=1, n_heads=2, n_kv_heads=2, head_dim=2, vocab=4, ffn_inter=4)
    I4 = np.eye(4, dtype=np.float32)
    embed = np.zeros((4, 4), np.float32)
    embed[0] = [1.0, 0, 0, 0]
    w_qkv = np.concatenate([w_q, np.zeros((8, 4), np.float32)])
    W = {"embed": bits(embed), "lm_head": bits(I4), "final_norm": np.ones(4, np.float32),
         "layers": [{"attn_norm": np.ones(4, np.float32), "ffn_norm": np.ones(4, np.float32),
                     "w_qkv": bits(w_qkv), "w_o": bits(I4), "w_gate_up": bits(np.zeros((8, 4), np.float32)),
                     "w_down": bits(np.zeros((4, 4), np.float32))}]}
    return s, W


def _norm_logits(x1, eps):
    x1 = np.asarray(x1, dtype=np.float64)
    return x1 / math.sqrt(float(np.mean(x1 * x1)) + eps)


def test_kv_load_values_and_length():
    """A loaded prefix is the cache (decoder.rs: a prefix restore uploads
    host K/V rows into the resident cache): with W_q = 0 every score is 0, so
    each head's output is the mean of its kv head's V rows over the two loaded
    positions and the query's own (zero) value.  V is [Hkv][len][d]: a
    position-major reading or a swapped head would change the mean."""
    s, W = _kv_load_model(np.zeros((4, 4), np.float32))
    m = oracle.Model(s, W)
    V = np.array([[[1.0, 2.0], [3.0, -4.0]],          # kv head 0: positions 0, 1
                  [[0.5, 8.0], [-6.0, 0.25]]], np.float32)
    K = np.array([[[7.0, -1.0], [2.0, 3.0]], [[-5.0, 1.5], [4.0, 0.5]]], np.float32)
    m.kv_load(0, 0, bits(K), bits(V), 2)
    assert m.seq_len(0) == 2
    with pytest.raises(oracle.OracleError):
        m.forward([0], 1)                              # the next position is 2
    lg = m.forward([0], 2)["logits"]
    V64 = V.astype(np.float64)
    out = np.concatenate([(V64[0, 0] + V64[0, 1]) / 3.0, (V64[1, 0] + V64[1, 1]) / 3.0])
    want = _norm_logits(np.array([1.0, 0, 0, 0]) + out, s.rms_eps)
    assert np.allclose(lg, want, rtol=1e-13, atol=1e-15)


def test_kv_load_keys_select_their_value():
    """One loaded key per head dominates its head's softmax, so the head's
    output is that key's V row: head 0 is steered to position 1 and head 1 to
    position 0 through K alone.  The query q_h = (a_0, 0) of both heads is
    rotated at position 2 by 2 radians (d = 2: theta_0 = 1), and each chosen
    key points along it with length 200, a score of about 283 against 0 for the
    other keys.  K read with heads and positions swapped selects the wrong
    rows."""
    w_q = np.zeros((4, 4), np.float32)
    w_q[0, 0] = 1.0        # head 0: q = (a_0, 0)
    w_q[2, 0] = 1.0        # head 1: q = (a_0, 0)
    s, W = _kv_load_model(w_q)
    m = oracle.Model(s, W)
    k = 200.0 * np.array([math.cos(2.0), math.sin(2.0)])
    kb = synth.bf16_to_f32(np.array([synth.f32_to_bf16(v) for v in k], np.uint16))
    K = np.zeros((2, 2, 2), np.float32)
    K[0, 1] = kb            # head 0 -> position 1
    K[1, 0] = kb            # head 1 -> position 0
    V = np.array([[[1.0, 2.0], [3.0, -4.0]], [[0.5, 8.0], [-6.0, 0.25]]], np.float32)
    m.kv_load(0, 0, bits(K), bits(V), 2)
    lg = m.forward([0], 2)["logits"]
    out = np.concatenate([V[0, 1], V[1, 0]]).astype(np.float64)
    want = _norm_logits(np.array([1.0, 0, 0, 0]) + out, s.rms_eps)
    assert np.allclose(lg, want, rtol=1e-13, atol=1e-15)


def test_kv_load_errors():
    s, W = _kv_load_model(np.zeros((4, 4), np.float32))
    m = oracle.Model(s, W)
    z = np.zeros((2, 40, 2), np.uint16)
    with pytest.raises(oracle.OracleError):
        m.kv_load(0, 0, z, z, s.max_seq + 1)           # past max_seq
    with pytest.raises(oracle.OracleError):
        m.kv_load(0, 1, z, z, 2)                       # no layer 1


def test_reset_equals_a_fresh_model():
    """engine.zig Engine.reset forgets the cache: after a reset, a sequence
    computes bit for bit what a fresh model computes, and resetting one
    sequence leaves another untouched."""
    s = small_shape()
    W = rand_weights(s)
    a_ids, b_ids = synth.tokens(9, 11, s.vocab), synth.tokens(7, 12, s.vocab)
    fresh = oracle.Model(s, W).forward(a_ids, 0, logits_mode=2)["logits"]
    m = oracle.Model(s, W, n_seqs=2)
    m.forward(b_ids, 0, seq=0, logits_mode=0)
    m.forward(a_ids[:4], 0, seq=1, logits_mode=0)
    m.reset(0)
    assert m.seq_len(0) == 0 and m.seq_len(1) == 4
    got = m.forward(a_ids, 0, seq=0, logits_mode=2)["logits"]
    assert np.array_equal(got, fresh)
    # seq 1 kept its 4 positions: its continuation equals an unbroken run
    tail = m.forward(a_ids[4:], 4, seq=1, logits_mode=2)["logits"]
    assert np.array_equal(tail, fresh[4:])
    m.reset(-1)
    assert m.seq_len(0) == 0 and m.seq_len(1) == 0
    assert np.array_equal(m.forward(a_ids, 0, seq=1, logits_mode=2)["logits"], fresh)


def test_decode_after_prefill_equals_recompute():
    s = small_shape()
    W = rand_weights(s)
    ids = synth.tokens(12, 5, s.vocab)
    m = oracle.Model(s, W)
    m.forward(ids[:8], 0, logits_mode=0)
    step = [m.forward(ids[8 + i:9 + i], 8 + i)["logits"] for i in range(4)]
    full = oracle.Model(s, W).forward(ids, 0, logits_mode=2)["logits"]
    for i in range(4):
        assert np.allclose(step[i], full[8 + i], rtol=0, atol=1e-12)


def test_truncate_equals_never_extended():
    """Rolling a sequence back (pipeline.rs Pipeline::generate_from_ids
    drops a rejected draft's KV entry) leaves exactly the state of a sequence
    that never held the dropped rows.  A slip in the rolled-back length (one
    row too many or too few) changes the next token's attention keys."""
    s = small_shape()
    W = rand_weights(s)
    ids = synth.tokens(14, 9, s.vocab)
    a = oracle.Model(s, W)
    a.forward(ids[:8], 0, logits_mode=0)
    a.forward(ids[8:12], 8, logits_mode=2)          # four drafted positions
    a.truncate(0, 9)                                # keep one of them
    assert a.seq_len(0) == 9
    got = a.forward(ids[12:13], 9)["logits"]
    b = oracle.Model(s, W)
    b.forward(ids[:9], 0, logits_mode=0)
    want = b.forward(ids[12:13], 9)["logits"]
    assert np.array_equal(got, want)
    c = oracle.Model(s, W)                          # keeping all four differs
    c.forward(ids[:12], 0, logits_mode=0)
    assert not np.allclose(c.forward(ids[12:13], 12)["logits"], want)
    with pytest.raises(ValueError):
        a.truncate(0, 11)                           # past the current length


def test_chunk_size_invariance():
    s = small_shape()
    W = rand_weights(s)
    ids = synth.tokens(16, 11, s.vocab)
    ref = oracle.Model(s, W).prefill(ids, 16)["logits"]
    for chunk in (1, 3, 5):
        got = oracle.Model(s, W).prefill(ids, chunk)["logits"]
        assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_causality():
    s = small_shape()
    W = rand_weights(s)
    ids = synth.tokens(10, 3, s.vocab)
    a = oracle.Model(s, W).forward(ids, 0, logits_mode=2)["logits"]
    ids2 = ids.copy()
    ids2[6:] = (ids2[6:] + 1) % s.vocab
    b = oracle.Model(s, W).forward(ids2, 0, logits_mode=2)["logits"]
    assert np.array_equal(a[:6], b[:6])
    assert not np.allclose(a[6:], b[6:])


def test_gqa_model_equals_mha_model_with_repeated_kv_rows():
    s = small_shape(n_heads=4, n_kv_heads=2)
    W = rand_weights(s)
    d, Hq, Hkv = s.head_dim, s.n_heads, s.n_kv_heads
    s_mha = small_shape(n_heads=4, n_kv_heads=4)
    W2 = {k: v for k, v in W.items() if k != "layers"}
    W2["layers"] = []
    rep = Hq // Hkv
    for L in W["layers"]:
        q = L["w_qkv"][:Hq * d]
        k = L["w_qkv"][Hq * d:(Hq + Hkv) * d].reshape(Hkv, d, -1)
        v = L["w_qkv"][(Hq + Hkv) * d:].reshape(Hkv, d, -1)
        k = np.repeat(k, rep, axis=0).reshape(Hq * d, -1)
        v = np.repeat(v, rep, axis=0).reshape(Hq * d, -1)
        L2 = dict(L)
        L2["w_qkv"] = np.ascontiguousarray(np.concatenate([q, k, v]))
        W2["layers"].append(L2)
    ids = synth.tokens(9, 21, s.vocab)
    a = oracle.Model(s, W).forward(ids, 0, logits_mode=2)["logits"]
    b = oracle.Model(s_mha, W2).forward(ids, 0, logits_mode=2)["logits"]
    assert np.allclose(a, b, rtol=0, atol=1e-13)


# -------------------------------------------------------------------- MoE --

def moe_shape(**kw):
    base = dict(hidden=32, n_layers=1, n_heads=2, n_kv_heads=2, head_dim=8, vocab=64,
                n_experts=4, top_k=2, expert_inter=12, shared_inter=0, ffn_inter=0)
    base.update(kw)
    return small_shape(**base)


def dense_from(W_moe, gate_up, down):
    W = {k: v for k, v in W_moe.items() if k != "layers"}
    L = {k: W_moe["layers"][0][k] for k in ("attn_norm", "ffn_norm", "w_qkv", "w_o") if k in W_moe["layers"][0]}
    L["w_gate_up"], L["w_down"] = np.ascontiguousarray(gate_up), np.ascontiguousarray(down)
    W["layers"] = [L]
    return W


def test_moe_all_experts_uniform_gate_equals_dense_average():
    E, Ie = 4, 12
    s = moe_shape(top_k=E)
    W = rand_weights(s)
    L = W["layers"][0]
    L["w_router"] = bits(np.zeros((E, s.hidden), np.float32))      # P = 1/E for every expert
    g = L["w_exp_gate_up"][:, :Ie]
    u = L["w_exp_gate_up"][:, Ie:]
    gate_up = np.concatenate([g.reshape(E * Ie, -1), u.reshape(E * Ie, -1)])
    down = np.concatenate([L["w_exp_down"][e] for e in range(E)], axis=1)
    down_avg = bits(widen(down) / E)                                 # exact: E is a power of two
    sd = small_shape(hidden=32, n_layers=1, n_heads=2, n_kv_heads=2, head_dim=8, vocab=64,
                     ffn_inter=E * Ie)
    ids = synth.tokens(7, 2, s.vocab)
    a = oracle.Model(s, W).forward(ids, 0, logits_mode=2)["logits"]
    b = oracle.Model(sd, dense_from(W, gate_up, down_avg)).forward(ids, 0, logits_mode=2)["logits"]
    assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_moe_top1_renormalised_equals_that_expert():
    s = moe_shape(top_k=1, norm_topk_prob=1)
    W = rand_weights(s)
    L = W["layers"][0]
    L["w_router"] = bits(np.zeros((s.n_experts, s.hidden), np.float32))  # tie -> expert 0
    sd = small_shape(hidden=32, n_layers=1, n_heads=2, n_kv_heads=2, head_dim=8, vocab=64,
                     ffn_inter=s.expert_inter)
    ids = synth.tokens(6, 4, s.vocab)
    out = oracle.Model(s, W).forward(ids, 0, logits_mode=2, routes=True)
    assert np.all(out["routes"] == 0)
    b = oracle.Model(sd, dense_from(W, L["w_exp_gate_up"][0], L["w_exp_down"][0])).forward(
        ids, 0, logits_mode=2)["logits"]
    assert np.allclose(out["logits"], b, rtol=0, atol=1e-12)


@pytest.mark.parametrize("with_gate", [True, False])
def test_moe_shared_expert_gate_scale(with_gate):
    # routed experts zero: the output comes from the shared expert alone, at
    # x0.5 when the gate vector is zero (sigmoid(0)) and x1 when it is absent.
    s = moe_shape(shared_inter=16, shared_gate=with_gate)
    W = rand_weights(s)
    L = W["layers"][0]
    L["w_exp_gate_up"] = np.zeros_like(L["w_exp_gate_up"])
    L["w_exp_down"] = np.zeros_like(L["w_exp_down"])
    if with_gate:
        L["w_sh_gate"] = bits(np.zeros(s.hidden, np.float32))
    scale = 0.5 if with_gate else 1.0
    sd = small_shape(hidden=32, n_layers=1, n_heads=2, n_kv_heads=2, head_dim=8, vocab=64,
                     ffn_inter=16)
    ids = synth.tokens(5, 8, s.vocab)
    a = oracle.Model(s, W).forward(ids, 0, logits_mode=2)["logits"]
    down = bits(widen(L["w_sh_down"]) * scale)
    b = oracle.Model(sd, dense_from(W, L["w_sh_gate_up"], down)).forward(ids, 0, logits_mode=2)["logits"]
    assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_moe_routes_are_distinct_and_chunk_invariant():
    s = moe_shape(n_experts=8, top_k=3, shared_inter=16, shared_gate=True, qkv_bias=True, n_layers=2)
    W = rand_weights(s)
    ids = synth.tokens(12, 13, s.vocab)
    full = oracle.Model(s, W).forward(ids, 0, logits_mode=2, routes=True)
    for l in range(s.n_layers):
        for i in range(12):
            assert len(set(full["routes"][l, i])) == 3
    m = oracle.Model(s, W)
    step = [m.forward(ids[i:i + 1], i, routes=True) for i in range(12)]
    for i in range(12):
        assert np.allclose(step[i]["logits"], full["logits"][i], rtol=0, atol=1e-12)
        assert np.array_equal(step[i]["routes"][:, 0], full["routes"][:, i])


@pytest.mark.parametrize("renorm", [0, 1])
def test_moe_forced_routes(renorm):
    """Teacher-forced expert ids (the oracle follows a given expert set where
    two are correct): with a zero router every probability is 1/E, so
    forcing experts {3, 1} must equal a dense SwiGLU made of those two
    experts with the down rows scaled by their weight, 1/E, or 1/2 when
    the top-k is renormalised (both exact: powers of two).  Forcing the
    oracle's own choice changes nothing, and invalid sets are refused."""
    E, Ie = 4, 12
    s = moe_shape(top_k=2, norm_topk_prob=renorm, n_layers=1)
    W = rand_weights(s)
    ids = synth.tokens(6, 21, s.vocab)
    own = oracle.Model(s, W).forward(ids, 0, logits_mode=2, routes=True)
    again = oracle.Model(s, W).forward(ids, 0, logits_mode=2, force_routes=own["routes"])
    assert np.array_equal(own["logits"], again["logits"])
    L = W["layers"][0]
    L["w_router"] = bits(np.zeros((E, s.hidden), np.float32))
    force = np.tile(np.array([3, 1], np.int32), (1, 6, 1))
    a = oracle.Model(s, W).forward(ids, 0, logits_mode=2, force_routes=force, routes=True)
    assert np.all(a["routes"] == force)
    sel = [3, 1]
    g = np.concatenate([L["w_exp_gate_up"][e][:Ie] for e in sel])
    u = np.concatenate([L["w_exp_gate_up"][e][Ie:] for e in sel])
    down = np.concatenate([L["w_exp_down"][e] for e in sel], axis=1)
    w = 0.5 if renorm else 1.0 / E
    sd = small_shape(hidden=32, n_layers=1, n_heads=2, n_kv_heads=2, head_dim=8, vocab=64, ffn_inter=2 * Ie)
    b = oracle.Model(sd, dense_from(W, np.concatenate([g, u]), bits(widen(down) * w))).forward(
        ids, 0, logits_mode=2)["logits"]
    assert np.allclose(a["logits"], b, rtol=0, atol=1e-12)
    for bad in ([1, 1], [0, E]):
        with pytest.raises(oracle.OracleError):
            oracle.Model(s, W).forward(ids, 0, logits_mode=2,
                                       force_routes=np.tile(np.array(bad, np.int32), (1, 6, 1)))


# ----------------------------------------------------------------- errors --

def test_boundary_errors():
    s = small_shape(max_seq=8)
    m = oracle.Model(s, rand_weights(s))
    with pytest.raises(oracle.OracleError, match="token"):
        m.forward([s.vocab], 0)
    with pytest.raises(oracle.OracleError, match="overflow"):
        m.forward(list(range(9)), 0)
    m.forward(list(range(8)), 0)              # exactly filling the cache is allowed
    with pytest.raises(oracle.OracleError, match="overflow"):
        m.forward([1], 8)
    with pytest.raises(oracle.OracleError, match="invalid"):
        oracle.Model(s, rand_weights(s)).forward([1], 3)   # start_pos must equal the length


# ------------------------------------------------------------- bf16 KV --

def test_round_bf16_matches_rne_reference():
    # exact on fp32 inputs: the result must equal the bit-level fp32 -> bf16
    # round-to-nearest-even of the generator (a separate implementation)
    vals = np.random.default_rng(5).normal(size=2000).astype(np.float32) * np.float32(3.7)
    for v in vals:
        want = synth.bf16_to_f32(np.array([synth.f32_to_bf16(float(v))], np.uint16))[0]
        assert oracle.round_bf16(float(v)) == float(want)
    assert oracle.round_bf16(1.0 + 2 ** -8) == 1.0                 # tie -> even
    assert oracle.round_bf16(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6   # tie -> even (up)
    assert oracle.round_bf16(-(1.0 + 2 ** -8 + 2 ** -30)) == -(1.0 + 2 ** -7)
    assert oracle.round_bf16(0.0) == 0.0


def test_bf16_kv_cache_rounds_only_the_cache():
    # with one cached position the attention output is v itself, so x after
    # the layer carries exactly the bf16 rounding of v (and nothing else)
    s = small_shape(hidden=4, n_layers=1, n_heads=1, n_kv_heads=1, head_dim=4, vocab=4,
                    ffn_inter=4, qkv_bias=True)
    I4 = np.eye(4, dtype=np.float32)
    bias = np.zeros(12, np.float32)
    bias[8:12] = [0.5, -1.0, 0.25, 2.0]
    w_qkv = np.zeros((12, 4), np.float32)
    w_qkv[8:12] = I4 * np.float32(1.0 + 2 ** -7)     # v = 1.0078125 * a + b_v
    embed = np.zeros((4, 4), np.float32)
    embed[0] = [1.0, 0, 0, 0]
    W = {"embed": bits(embed), "lm_head": bits(I4), "final_norm": np.ones(4, np.float32),
         "layers": [{"attn_norm": np.ones(4, np.float32), "ffn_norm": np.ones(4, np.float32),
                     "w_qkv": bits(w_qkv), "b_qkv": bias,
                     "w_o": bits(I4), "w_gate_up": bits(np.zeros((8, 4), np.float32)),
                     "w_down": bits(np.zeros((4, 4), np.float32))}]}
    a0 = 2.0 / math.sqrt(1.0 + 4 * s.rms_eps)         # x = (1,0,0,0): mean(x^2) = 1/4
    v_exact = np.array([(1 + 2 ** -7) * a0 + 0.5, -1.0, 0.25, 2.0])
    x_exact = oracle.Model(s, W, kv_bf16=False).forward([0], 0, trace=True)["trace"][1, 0]
    x_bf = oracle.Model(s, W, kv_bf16=True).forward([0], 0, trace=True)["trace"][1, 0]
    assert np.allclose(x_exact, np.array([1.0, 0, 0, 0]) + v_exact, atol=1e-15)
    assert np.allclose(x_bf, np.array([1.0, 0, 0, 0]) + [oracle.round_bf16(t) for t in v_exact], atol=1e-15)
    assert not np.allclose(x_exact, x_bf, atol=1e-6)


# ------------------------------------------------------ weight quantisation --

def test_quantize_rows_worked_example():
    """int8 codes with a power-of-two scale per row: row 0 has largest
    magnitude 1, so 127 * 2^e >= 1 first holds at e = -6 (codes 64, -32, 16,
    and 0.0078125 * 64 = 0.5 rounds to the even 0); row 1's largest magnitude
    0.3125 gives e = -8 (127 / 256 >= 0.3125 > 127 / 512), and 0.3828125 *
    256 = 98 exactly; row 2 checks the tie 1.5 -> 2 and -2.5 -> -2."""
    W = bits(np.array([[1.0, -0.5, 0.25, 0.0078125],
                       [0.3125, -0.0625, 0.3828125, 0.015625],
                       [1.5 / 64, -2.5 / 64, 1.0, 0.0]], np.float32))
    deq, e = oracle.quantize_rows(W, 3, 4)
    got = synth.bf16_to_f32(deq)
    assert list(e) == [-6, -8, -6]
    assert np.array_equal(got[0], np.array([1.0, -0.5, 0.25, 0.0], np.float32))
    assert np.array_equal(got[1], np.array([0.3125, -0.0625, 0.3828125, 0.015625], np.float32))
    assert np.array_equal(got[2], np.array([2 / 64, -2 / 64, 1.0, 0.0], np.float32))


def test_quantize_rows_properties():
    rows, K = 64, 96
    W = rand_bits((rows, K), 0.05)
    w = widen(W)
    deq, e = oracle.quantize_rows(W, rows, K)
    d = widen(deq)
    step = np.ldexp(1.0, e)[:, None]
    q = d / step
    assert np.array_equal(q, np.rint(q))                      # integer codes
    assert np.abs(q).max() <= 127                             # in int8 range
    assert np.all(np.abs(q).max(axis=1) >= 64)                # e is the smallest that covers the row
    assert np.all(np.abs(w - d) <= step / 2)                  # rounded to the nearest code
    again, e2 = oracle.quantize_rows(deq, rows, K)            # idempotent
    assert np.array_equal(again, deq) and np.array_equal(e2, e)


def test_quantize_q4_worked_example():
    """4-bit codes with a power-of-two scale per group of 32 weights.
    Row 0, group 0: largest magnitude 1.75, and 7 * 2^e >= 1.75 first holds
    at e = -2 (step 0.25): codes 7, -2, 1, 0.5 -> 0 and 1.5 -> 2 (ties to
    even), -2.5 -> -2, 1.25 -> 1.  Group 1: largest 3/128, e = -8 (7/256
    covers it, 7/512 does not): codes 6 and -3.  Group 2 is all zero: e = 0.
    Row 1 sits on the boundary: a group whose largest magnitude is exactly
    7 * 2^-5 takes e = -5 (code 7); the next bf16 value up, 0.2197265625,
    needs e = -4 and becomes code 4 (3.515625 rounded)."""
    W = np.zeros((2, 96), np.float32)
    W[0, :7] = [1.75, -0.5, 0.25, 0.125, 0.375, -0.625, 0.3125]
    W[0, 32:34] = [3 / 128, -3 / 256]
    W[1, 0] = 0.21875
    W[1, 32] = 0.2197265625
    deq, q, e = oracle.quantize_q4(bits(W), 2, 96)
    assert e.tolist() == [[-2, -8, 0], [-5, -4, 0]]
    assert q[0, :7].tolist() == [7, -2, 1, 0, 2, -2, 1]
    assert q[0, 32:34].tolist() == [6, -3]
    assert q[1, 0] == 7 and q[1, 32] == 4
    got = synth.bf16_to_f32(deq)
    assert np.array_equal(got[0, :7], np.array([1.75, -0.5, 0.25, 0.0, 0.5, -0.5, 0.25], np.float32))
    assert got[1, 32] == 0.25
    assert np.count_nonzero(q) == 10


def test_quantize_q4_properties():
    rows, K = 48, 128
    W = rand_bits((rows, K), 0.05)
    w = widen(W)
    deq, q, e = oracle.quantize_q4(W, rows, K)
    d = widen(deq)
    step = np.repeat(np.ldexp(1.0, e), 32, axis=1)
    assert np.array_equal(d, q.astype(np.float64) * step)       # deq = code x 2^e exactly
    assert np.abs(q).max() <= 7                                  # 4-bit signed range
    gmax = np.abs(q).reshape(rows, K // 32, 32).max(axis=2)
    assert np.all(gmax >= 4)                                     # e is the smallest that covers the group
    assert np.all(np.abs(w - d) <= step / 2)                     # rounded to the nearest code
    again, q2, e2 = oracle.quantize_q4(deq, rows, K)             # idempotent
    assert np.array_equal(again, deq) and np.array_equal(q2, q) and np.array_equal(e2, e)
