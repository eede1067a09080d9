"""Python binding of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It imports nothing from the GPU package.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_D = ctypes.c_double


class OrcConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden", "n_layers", "n_heads", "n_kv_heads", "head_dim", "ffn_inter", "n_experts",
        "top_k", "expert_inter", "shared_inter", "norm_topk_prob", "vocab", "qkv_bias")] + [
        ("rope_base", ctypes.c_double), ("rms_eps", ctypes.c_double),
        ("max_seq", ctypes.c_int32), ("n_seqs", ctypes.c_int32), ("kv_bf16", ctypes.c_int32),
        ("sliding_window", ctypes.c_int32), ("attn_softcap", ctypes.c_double), ("qk_norm", ctypes.c_int32)]


LAYER_FIELDS = ("attn_norm", "ffn_norm", "w_qkv", "b_qkv", "w_o", "w_gate_up", "w_down",
                "w_router", "w_exp_gate_up", "w_exp_down", "w_sh_gate_up", "w_sh_down",
                "w_sh_gate", "attn_sinks", "q_norm", "k_norm")


class OrcLayer(ctypes.Structure):
    _fields_ = [(n, _P) for n in LAYER_FIELDS]


class OrcWeights(ctypes.Structure):
    _fields_ = [("embed", _P), ("final_norm", _P), ("lm_head", _P), ("layers", ctypes.POINTER(OrcLayer))]


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(path)
        L.orc_num_threads.restype = _I
        L.orc_round_bf16.restype = _D
        L.orc_round_bf16.argtypes = [_D]
        L.orc_rmsnorm.argtypes = [_P, _P, _I, _D, _P]
        L.orc_matmul.argtypes = [_P, _I, _I, _P, _I, _P]
        L.orc_matvec.argtypes = [_P, _I, _I, _P, _P]
        L.orc_rope.argtypes = [_P, _I, _I, ctypes.c_long, _D]
        L.orc_attend.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _D, _P, _P]
        L.orc_silu.restype = _D
        L.orc_silu.argtypes = [_D]
        L.orc_sigmoid.restype = _D
        L.orc_sigmoid.argtypes = [_D]
        L.orc_route.argtypes = [_P, _I, _I, _I, _P, _P, _P]
        L.orc_argmax.restype = ctypes.c_int32
        L.orc_argmax.argtypes = [_P, _I]
        L.orc_create.restype = _P
        L.orc_create.argtypes = [ctypes.POINTER(OrcConfig), ctypes.POINTER(OrcWeights)]
        L.orc_free.argtypes = [_P]
        L.orc_reset.argtypes = [_P, _I]
        L.orc_kv_load.restype = _I
        L.orc_kv_load.argtypes = [_P, _I, _I, _P, _P, _I]
        L.orc_quantize_rows.restype = None
        L.orc_quantize_rows.argtypes = [_P, _I, _I, _P, _P]
        L.orc_quantize_q4.restype = None
        L.orc_quantize_q4.argtypes = [_P, _I, _I, _P, _P, _P]
        L.orc_truncate.restype = _I
        L.orc_truncate.argtypes = [_P, _I, _I]
        L.orc_seq_len.restype = ctypes.c_int32
        L.orc_seq_len.argtypes = [_P, _I]
        L.orc_forward.restype = _I
        L.orc_forward.argtypes = [_P, _I, _P, _I, _I, _I, _P, _P, _P, _P, _P]
        _LIB = L
    return _LIB


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def num_threads():
    return lib().orc_num_threads()


def round_bf16(v):
    return lib().orc_round_bf16(float(v))


# ------------------------------------------------------------ primitives --

def rmsnorm(x, g, eps):
    x = _f64(x)
    g = np.ascontiguousarray(g, dtype=np.float32)
    out = np.empty_like(x)
    lib().orc_rmsnorm(x.ctypes.data, g.ctypes.data, x.size, float(eps), out.ctypes.data)
    return out


def matmul(W_bits, rows, cols, X):
    """Y[i] = W X[i] for bf16 W (uint16 bits, [rows][cols]) and fp64 X ([n][cols])."""
    W_bits = np.ascontiguousarray(W_bits, dtype=np.uint16)
    X = _f64(X).reshape(-1, cols)
    Y = np.empty((X.shape[0], rows), dtype=np.float64)
    lib().orc_matmul(W_bits.ctypes.data, rows, cols, X.ctypes.data, X.shape[0], Y.ctypes.data)
    return Y


def rope(v, nheads, d, pos, base):
    v = _f64(v).copy()
    lib().orc_rope(v.ctypes.data, nheads, d, int(pos), float(base))
    return v


def attend(q, kc, vc, Hq, Hkv, d, window=0, softcap=0.0, sinks=None):
    """q [Hq*d]; kc, vc [T][Hkv*d] -> out [Hq*d].  window, softcap and sinks
    ([Hq] fp32) select the attention variants (0 / None: off)."""
    q, kc, vc = _f64(q), _f64(kc), _f64(vc)
    T = kc.size // (Hkv * d)
    out = np.empty(Hq * d, dtype=np.float64)
    sk = None if sinks is None else np.ascontiguousarray(sinks, dtype=np.float32)
    lib().orc_attend(q.ctypes.data, kc.ctypes.data, vc.ctypes.data, T, Hq, Hkv, d, int(window),
                     float(softcap), None if sk is None else sk.ctypes.data, out.ctypes.data)
    return out


def silu(z):
    return lib().orc_silu(float(z))


def sigmoid(z):
    return lib().orc_sigmoid(float(z))


def route(logits, k, renorm):
    logits = _f64(logits)
    E = logits.size
    idx = np.empty(k, dtype=np.int32)
    w = np.empty(k, dtype=np.float64)
    p = np.empty(E, dtype=np.float64)
    lib().orc_route(logits.ctypes.data, E, k, int(renorm), idx.ctypes.data, w.ctypes.data, p.ctypes.data)
    return idx, w, p


def argmax(v):
    v = _f64(v)
    return int(lib().orc_argmax(v.ctypes.data, v.size))


def quantize_rows(W_bits, rows, cols):
    """int8 codes with one power-of-two scale per row, returned dequantised
    (bf16 bit patterns, exact) together with the per-row exponents."""
    W_bits = np.ascontiguousarray(W_bits, dtype=np.uint16).reshape(rows, cols)
    out = np.empty_like(W_bits)
    e = np.empty(rows, dtype=np.int32)
    lib().orc_quantize_rows(W_bits.ctypes.data, rows, cols, out.ctypes.data, e.ctypes.data)
    return out, e


def quantize_q4(W_bits, rows, cols):
    """4-bit codes with one power-of-two scale per group of 32 weights:
    returns the dequantised weights (bf16 bit patterns, exact), the codes
    [rows][cols] (int8 values in [-7, 7]) and the exponents [rows][cols / 32]."""
    W_bits = np.ascontiguousarray(W_bits, dtype=np.uint16).reshape(rows, cols)
    out = np.empty_like(W_bits)
    q = np.empty((rows, cols), dtype=np.int8)
    e = np.empty((rows, cols // 32), dtype=np.int32)
    lib().orc_quantize_q4(W_bits.ctypes.data, rows, cols, out.ctypes.data, q.ctypes.data, e.ctypes.data)
    return out, q, e


def quant_dims(shape):
    """(rows, cols) of every matrix the quantised decoder streams as int8
    rows: the attention projections, the dense or shared-expert FFN, and
    every routed expert's rows (the router and the shared gate stay bf16)."""
    s = shape
    H = s.hidden
    dims = {"w_qkv": (s.qkv_rows, H), "w_o": (H, s.q_dim)}
    if s.is_moe:
        E, Ie, Is = s.n_experts, s.expert_inter, s.shared_inter
        dims.update(w_exp_gate_up=(E * 2 * Ie, H), w_exp_down=(E * H, Ie))
        if Is:
            dims.update(w_sh_gate_up=(2 * Is, H), w_sh_down=(H, Is))
    else:
        dims.update(w_gate_up=(2 * s.ffn_inter, H), w_down=(H, s.ffn_inter))
    return dims


def quantized_weights(shape, weights):
    """The model's weights as the quantised decoder holds them: those
    matrices and the lm-head dequantised (the embedding gather keeps its
    bf16 table).  weight_quant 1: int8 codes, one scale per row; 2: 4-bit
    codes, one scale per group of 32 weights."""
    s = shape
    H = s.hidden
    dims = quant_dims(s)
    q = (lambda W, r, c: quantize_rows(W, r, c)[0]) if s.weight_quant == 1 else \
        (lambda W, r, c: quantize_q4(W, r, c)[0])
    out = dict(weights)
    out["layers"] = []
    for L in weights["layers"]:
        L2 = dict(L)
        for f, (r, c) in dims.items():
            L2[f] = q(L[f], r, c).reshape(-1)
        out["layers"].append(L2)
    out["lm_head"] = q(weights["lm_head"], s.vocab, H).reshape(-1)
    return out


# ----------------------------------------------------------------- model --

class OracleError(RuntimeError):
    pass


ERRORS = {1: "context overflow", 2: "invalid argument", 3: "token out of range", 4: "out of memory"}


class Model:
    """fp64 reference decoder over host weights from synth.weights.host_weights.

    kv_bf16 (default: the shape's kv_bf16) stores the KV cache as bf16 values."""

    def __init__(self, shape, weights, n_seqs=1, max_seq=None, kv_bf16=None):
        self.shape = shape
        if getattr(shape, "weight_quant", 0):
            weights = quantized_weights(shape, weights)
        self._keep = []
        s = shape
        cfg = OrcConfig(hidden=s.hidden, n_layers=s.n_layers, n_heads=s.n_heads,
                        n_kv_heads=s.n_kv_heads, head_dim=s.head_dim, ffn_inter=s.ffn_inter,
                        n_experts=s.n_experts, top_k=s.top_k, expert_inter=s.expert_inter,
                        shared_inter=s.shared_inter, norm_topk_prob=s.norm_topk_prob,
                        vocab=s.vocab, qkv_bias=int(s.qkv_bias), rope_base=s.rope_base,
                        rms_eps=s.rms_eps, max_seq=max_seq or s.max_seq, n_seqs=n_seqs,
                        kv_bf16=int(s.kv_bf16 if kv_bf16 is None else kv_bf16),
                        sliding_window=getattr(s, "sliding_window", 0),
                        attn_softcap=float(getattr(s, "attn_softcap", 0.0)),
                        qk_norm=int(getattr(s, "qk_norm", False)))
        self.max_seq = cfg.max_seq
        layers = (OrcLayer * s.n_layers)()
        for l in range(s.n_layers):
            for f in LAYER_FIELDS:
                arr = weights["layers"][l].get(f)
                if arr is not None:
                    arr = np.ascontiguousarray(arr)
                    self._keep.append(arr)
                    setattr(layers[l], f, arr.ctypes.data)
        self._keep.append(layers)
        w = OrcWeights()
        for f in ("embed", "final_norm", "lm_head"):
            arr = np.ascontiguousarray(weights[f])
            self._keep.append(arr)
            setattr(w, f, arr.ctypes.data)
        w.layers = layers
        self._cfg = cfg
        self._w = w
        self._h = lib().orc_create(ctypes.byref(cfg), ctypes.byref(w))
        if not self._h:
            raise OracleError("oracle allocation failed")

    def __del__(self):
        if getattr(self, "_h", None):
            lib().orc_free(self._h)
            self._h = None

    def reset(self, seq=-1):
        lib().orc_reset(self._h, seq)

    def truncate(self, seq, length):
        rc = lib().orc_truncate(self._h, seq, int(length))
        if rc != 0:
            raise ValueError(f"orc_truncate({seq}, {length}) failed: {rc}")

    def seq_len(self, seq=0):
        return lib().orc_seq_len(self._h, seq)

    def kv_load(self, seq, layer, K_bits, V_bits, length):
        K_bits = np.ascontiguousarray(K_bits, dtype=np.uint16)
        V_bits = np.ascontiguousarray(V_bits, dtype=np.uint16)
        rc = lib().orc_kv_load(self._h, seq, layer, K_bits.ctypes.data, V_bits.ctypes.data, length)
        if rc:
            raise OracleError(ERRORS.get(rc, rc))

    def forward(self, ids, start_pos, seq=0, logits_mode=1, routes=False, probs=False, trace=False,
                force_routes=None):
        """Forward a chunk; returns dict with 'logits' ([V] or [n][V]), 'routes', 'probs', 'trace'.
        force_routes ([L][n][k] int32): teacher-forced expert ids (each keeps
        its own softmax probability as its weight)."""
        s = self.shape
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        n = ids.size
        out = {}
        lg = None
        if logits_mode == 1:
            lg = np.empty(s.vocab, dtype=np.float64)
        elif logits_mode == 2:
            lg = np.empty((n, s.vocab), dtype=np.float64)
        rt = np.empty((s.n_layers, n, s.top_k), dtype=np.int32) if (routes and s.is_moe) else None
        pr = np.empty((s.n_layers, n, s.n_experts), dtype=np.float64) if (probs and s.is_moe) else None
        tr = np.empty((s.n_layers + 1, n, s.hidden), dtype=np.float64) if trace else None
        ptr = lambda a: a.ctypes.data if a is not None else None
        fr = None
        if force_routes is not None:
            fr = np.ascontiguousarray(force_routes, dtype=np.int32)
            assert fr.shape == (s.n_layers, n, s.top_k), fr.shape
        rc = lib().orc_forward(self._h, seq, ids.ctypes.data, n, int(start_pos), logits_mode,
                               ptr(lg), ptr(rt), ptr(pr), ptr(tr), ptr(fr))
        if rc:
            raise OracleError(ERRORS.get(rc, rc))
        out["logits"] = lg
        out["routes"] = rt
        out["probs"] = pr
        out["trace"] = tr
        return out

    def prefill(self, ids, chunk, seq=0, start_pos=0, **kw):
        """Prefill in chunks; returns the last chunk's forward() result (logits of the last token)."""
        res = None
        pos = start_pos
        for c0 in range(0, len(ids), chunk):
            part = ids[c0:c0 + chunk]
            res = self.forward(part, pos, seq=seq, logits_mode=1, **kw)
            pos += len(part)
        return res
