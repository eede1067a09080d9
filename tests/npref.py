"""An independent, vectorised numpy-float64 forward of the same block.

Cross-check for the C oracle (catches indexing slips in either): it shares
no code with oracle.c and processes a whole token sequence at once with a
causal mask instead of a growing cache.  Test infrastructure only.
"""
import numpy as np

import synth


def w(b):
    return synth.bf16_to_f32(b).astype(np.float64)


def rmsnorm(X, g, eps):
    return X / np.sqrt((X * X).mean(axis=-1, keepdims=True) + eps) * g.astype(np.float64)


def rope(T, pos, base):
    # T: [n, heads, d]; pairs (i, i + d/2) rotate by pos * base^(-2i/d)
    d = T.shape[-1]
    half = d // 2
    inv = base ** (-2.0 * np.arange(half) / d)
    ang = pos[:, None] * inv[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = T[..., :half], T[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def silu(z):
    return z / (1.0 + np.exp(-z))


def forward(shape, W, ids):
    """Logits [n][V] for every position of ids (fresh cache)."""
    s = shape
    H, Hq, Hkv, d = s.hidden, s.n_heads, s.n_kv_heads, s.head_dim
    n = len(ids)
    X = w(W["embed"]).reshape(s.vocab, H)[np.asarray(ids)]
    pos = np.arange(n, dtype=np.float64)
    mask = np.tril(np.ones((n, n), bool))
    for L in W["layers"]:
        A = rmsnorm(X, L["attn_norm"], s.rms_eps)
        QKV = A @ w(L["w_qkv"]).reshape(s.qkv_rows, H).T
        if s.qkv_bias:
            QKV = QKV + L["b_qkv"].astype(np.float64)
        Q = QKV[:, :Hq * d].reshape(n, Hq, d)
        K = QKV[:, Hq * d:(Hq + Hkv) * d].reshape(n, Hkv, d)
        if getattr(s, "qk_norm", False):
            Q = rmsnorm(Q, L["q_norm"], s.rms_eps)
            K = rmsnorm(K, L["k_norm"], s.rms_eps)
        Q = rope(Q, pos, s.rope_base)
        K = rope(K, pos, s.rope_base)
        V = QKV[:, (Hq + Hkv) * d:].reshape(n, Hkv, d)
        grp = Hq // Hkv
        K = np.repeat(K, grp, axis=1)
        V = np.repeat(V, grp, axis=1)
        S = np.einsum("ihd,jhd->hij", Q, K) / np.sqrt(d)
        cap = getattr(s, "attn_softcap", 0.0)
        if cap > 0:
            S = cap * np.tanh(S / cap)
        seen = mask
        win = getattr(s, "sliding_window", 0)
        if win > 0:
            seen = mask & (np.arange(n)[:, None] - np.arange(n)[None, :] < win)
        S = np.where(seen[None], S, -np.inf)
        sinks = L.get("attn_sinks")
        if sinks is not None:
            z = sinks.astype(np.float64)[:, None, None]
            top = np.maximum(S.max(axis=-1, keepdims=True), z)
            P = np.exp(S - top)
            P /= P.sum(axis=-1, keepdims=True) + np.exp(z - top)
        else:
            P = np.exp(S - S.max(axis=-1, keepdims=True))
            P /= P.sum(axis=-1, keepdims=True)
        O = np.einsum("hij,jhd->ihd", P, V).reshape(n, Hq * d)
        X = X + O @ w(L["w_o"]).reshape(H, Hq * d).T
        B = rmsnorm(X, L["ffn_norm"], s.rms_eps)
        if s.is_moe:
            E, k, Ie, Is = s.n_experts, s.top_k, s.expert_inter, s.shared_inter
            R = B @ w(L["w_router"]).reshape(E, H).T
            P = np.exp(R - R.max(axis=-1, keepdims=True))
            P /= P.sum(axis=-1, keepdims=True)
            order = np.argsort(-P, axis=-1, kind="stable")[:, :k]
            F = np.zeros_like(X)
            GU = w(L["w_exp_gate_up"]).reshape(E, 2 * Ie, H)
            DN = w(L["w_exp_down"]).reshape(E, H, Ie)
            for i in range(n):
                sel = order[i]
                wt = P[i, sel]
                if s.norm_topk_prob:
                    wt = wt / wt.sum()
                for e, we in zip(sel, wt):
                    gu = GU[e] @ B[i]
                    F[i] += we * (DN[e] @ (silu(gu[:Ie]) * gu[Ie:]))
            if Is:
                gu = B @ w(L["w_sh_gate_up"]).reshape(2 * Is, H).T
                Y = (silu(gu[:, :Is]) * gu[:, Is:]) @ w(L["w_sh_down"]).reshape(H, Is).T
                if s.shared_gate:
                    Y = Y / (1.0 + np.exp(-(B @ w(L["w_sh_gate"]))))[:, None]
                F += Y
            X = X + F
        else:
            I = s.ffn_inter
            gu = B @ w(L["w_gate_up"]).reshape(2 * I, H).T
            X = X + (silu(gu[:, :I]) * gu[:, I:]) @ w(L["w_down"]).reshape(H, I).T
    Xf = rmsnorm(X, W["final_norm"], s.rms_eps)
    return Xf @ w(W["lm_head"]).reshape(s.vocab, H).T
