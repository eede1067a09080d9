"""Which seed and scale every synthetic tensor is drawn with.

All matrices are bf16, row-major [out][in]:
  w_qkv    [(Hq + 2 Hkv) d][H]   q rows, then k rows, then v rows
  b_qkv    [(Hq + 2 Hkv) d]      fp32 holding bf16-rounded values
  w_o      [H][Hq d]
  w_gate_up[2 I][H]              gate rows, then up rows
  w_down   [H][I]
  w_router [E][H]
  w_exp_gate_up [E][2 Ie][H], w_exp_down [E][H][Ie]
  w_sh_gate_up [2 Is][H], w_sh_down [H][Is], w_sh_gate [H]
  attn_sinks [Hq]                fp32 holding bf16-rounded N(0, 1) values
  q_norm, k_norm [d]             fp32 1 + bf16-rounded N(0, 0.25^2) (per-head norm gains)
  embed, lm_head [V][H]; norm gains fp32 [H] equal to 1.0.
Matrices and biases are sigma = 0.02 normals; the router uses
sigma = 1/sqrt(H) so its logits over a unit-RMS input are about N(0, 1).
KV-cache fills are N(0, 1), laid out [Hkv][len][d] per (sequence, layer).
"""
import numpy as np

from . import normal_bf16, normal_bf16_f32, tensor_seed, tokens

WEIGHT_SEED = 20261202
PROMPT_SEED = 7
KV_SEED = 424242
SIGMA = 0.02

TID = dict(embed=1, lm_head=2, w_qkv=10, b_qkv=11, w_o=12, w_gate_up=13, w_down=14,
           w_router=15, w_exp_gate_up=16, w_exp_down=17, w_sh_gate_up=18, w_sh_down=19,
           w_sh_gate=20, attn_sinks=21, q_norm=22, k_norm=23)


def tensor_specs(shape):
    """[(name, layer or None, numel, sigma, kind)] for every generated tensor.
    kind is 'bf16' (matrix), 'f32' (bias stored as fp32), 'ones' (norm gain) or
    'gain' (fp32 1 + a bf16-rounded normal: the per-head q/k norm gains)."""
    s = shape
    H = s.hidden
    specs = [("embed", None, s.vocab * H, SIGMA, "bf16")]
    if not s.tied:
        specs.append(("lm_head", None, s.vocab * H, SIGMA, "bf16"))
    specs.append(("final_norm", None, H, 1.0, "ones"))
    for l in range(s.n_layers):
        specs += [("attn_norm", l, H, 1.0, "ones"), ("ffn_norm", l, H, 1.0, "ones"),
                  ("w_qkv", l, s.qkv_rows * H, SIGMA, "bf16")]
        if s.qkv_bias:
            specs.append(("b_qkv", l, s.qkv_rows, SIGMA, "f32"))
        specs.append(("w_o", l, H * s.q_dim, SIGMA, "bf16"))
        if s.attn_sinks:
            specs.append(("attn_sinks", l, s.n_heads, 1.0, "f32"))
        if s.qk_norm:
            specs += [("q_norm", l, s.head_dim, 0.25, "gain"), ("k_norm", l, s.head_dim, 0.25, "gain")]
        if s.is_moe:
            E, Ie, Is = s.n_experts, s.expert_inter, s.shared_inter
            specs += [("w_router", l, E * H, 1.0 / np.sqrt(H), "bf16"),
                      ("w_exp_gate_up", l, E * 2 * Ie * H, SIGMA, "bf16"),
                      ("w_exp_down", l, E * H * Ie, SIGMA, "bf16")]
            if Is:
                specs += [("w_sh_gate_up", l, 2 * Is * H, SIGMA, "bf16"),
                          ("w_sh_down", l, H * Is, SIGMA, "bf16")]
                if s.shared_gate:
                    specs.append(("w_sh_gate", l, H, SIGMA, "bf16"))
        else:
            specs += [("w_gate_up", l, 2 * s.ffn_inter * H, SIGMA, "bf16"),
                      ("w_down", l, H * s.ffn_inter, SIGMA, "bf16")]
    return specs


def seed_of(name, layer):
    return tensor_seed(WEIGHT_SEED, 0 if layer is None else layer, TID[name])


def host_tensor(name, layer, numel, sigma, kind):
    if kind == "ones":
        return np.ones(numel, dtype=np.float32)
    if kind == "f32":
        return normal_bf16_f32(numel, seed_of(name, layer), sigma)
    if kind == "gain":
        return normal_bf16_f32(numel, seed_of(name, layer), sigma) + np.float32(1.0)
    return normal_bf16(numel, seed_of(name, layer), sigma)


def host_weights(shape):
    """{'embed': u16[...], 'lm_head': ..., 'final_norm': f32, 'layers': [dict, ...]}."""
    out = {"layers": [dict() for _ in range(shape.n_layers)]}
    for name, layer, numel, sigma, kind in tensor_specs(shape):
        arr = host_tensor(name, layer, numel, sigma, kind)
        if layer is None:
            out[name] = arr
        else:
            out["layers"][layer][name] = arr
    if shape.tied:
        out["lm_head"] = out["embed"]
    return out


def prompt(shape, n, seq=0):
    return tokens(n, tensor_seed(PROMPT_SEED, seq, 99), shape.vocab)


def kv_seed(seq, layer, which):
    """which: 0 for K, 1 for V."""
    return tensor_seed(KV_SEED, layer, 2 * seq + which)


def host_kv(shape, seq, layer, length):
    n = shape.n_kv_heads * length * shape.head_dim
    return (normal_bf16(n, kv_seed(seq, layer, 0), 1.0),
            normal_bf16(n, kv_seed(seq, layer, 1), 1.0))
