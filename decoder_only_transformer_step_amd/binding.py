"""Thin ctypes binding of libdecoder.so (include/decoder.h, include/decoder_diag.h).

Argument marshalling only: PyTorch supplies device memory and the stream;
every step of the decoder runs in the library's HIP kernels.  The library
must have been built (``decoder_only_transformer_step_amd.build``); there is
no fallback path.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdecoder.so")
_LIB = None

DEC_OK, DEC_E_CONTEXT_OVERFLOW, DEC_E_INVALID, DEC_E_TOKEN, DEC_E_WORKSPACE, DEC_E_HIP = range(6)

_P = ctypes.c_void_p
_I32 = ctypes.c_int32


class DecoderConfig(ctypes.Structure):
    _fields_ = [(n, _I32) for n in (
        "hidden", "n_layers", "n_heads", "n_kv_heads", "head_dim", "ffn_inter", "n_experts",
        "top_k", "expert_inter", "shared_inter", "shared_gate", "norm_topk_prob", "vocab",
        "qkv_bias")] + [("rope_base", ctypes.c_double), ("rms_eps", ctypes.c_double)] + [
        (n, _I32) for n in ("max_seq", "max_chunk", "max_batch", "sliding_window")] + [
        ("attn_softcap", ctypes.c_double), ("qk_norm", _I32), ("weight_quant", _I32),
        ("kv_page_size", _I32), ("kv_pages", _I32)]


LAYER_FIELDS = ("attn_norm", "ffn_norm", "w_qkv", "b_qkv", "w_o", "w_gate_up", "w_down",
                "w_router", "w_exp_gate_up", "w_exp_down", "w_sh_gate_up", "w_sh_down",
                "w_sh_gate", "attn_sinks", "q_norm", "k_norm")


class DecoderLayerWeights(ctypes.Structure):
    _fields_ = [(n, _P) for n in LAYER_FIELDS]


class DecoderWeights(ctypes.Structure):
    _fields_ = [("embed", _P), ("final_norm", _P), ("lm_head", _P),
                ("layers", ctypes.POINTER(DecoderLayerWeights))]


NODES = ("qkv", "rope", "attn", "o", "gate_up", "down", "router", "experts", "head", "norm", "embed")


class DecoderStats(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64 * len(NODES)), ("ms", ctypes.c_double * len(NODES)),
                ("bytes", ctypes.c_double * len(NODES)), ("flops", ctypes.c_double * len(NODES))]

    def as_dict(self):
        return {n: dict(launches=int(self.launches[i]), ms=float(self.ms[i]), bytes=float(self.bytes[i]),
                        flops=float(self.flops[i])) for i, n in enumerate(NODES)}


# every symbol the headers declare, with its ctypes signature
SIGNATURES = {
    "decoder_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(DecoderConfig)]),
    "decoder_init": (ctypes.c_int, [ctypes.POINTER(DecoderConfig), ctypes.POINTER(DecoderWeights), _P,
                                    ctypes.c_size_t, _P, ctypes.POINTER(_P)]),
    "prefill_chunk": (ctypes.c_int, [_P, _I32, _P, _I32, _I32, _I32, _P, _P]),
    "decode_step": (ctypes.c_int, [_P, _I32, _P, _P, _P, _P]),
    "kv_reset": (ctypes.c_int, [_P, _I32]),
    "kv_truncate": (ctypes.c_int, [_P, _I32, _I32]),
    "decode_run": (ctypes.c_int, [_P, _I32, _I32, _P]),
    "kv_load": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _I32]),
    "decoder_seq_len": (_I32, [_P, _I32]),
    "decoder_set_stream": (ctypes.c_int, [_P, _P]),
    "decoder_free": (None, [_P]),
    "decoder_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "decoder_last_error": (ctypes.c_char_p, [_P]),
    "dec_diag_gemm": (ctypes.c_int, [_P, _I32, _I32, _P, _I32, _P, _P]),
    "dec_diag_gemm_chunk": (ctypes.c_int, [_P, _I32, _I32, _I32, _P, _I32, _P, _I32, _P, ctypes.c_int64, _P]),
    "dec_diag_gemm_grouped": (ctypes.c_int, [_P, _I32, _I32, _I32, _P, _I32, _I32, _P, _I32, _P, _P, _P]),
    "dec_diag_pack_w32": (ctypes.c_int, [_P, _I32, _I32, _P, _P]),
    "dec_diag_gemm_chunk_noalloc": (ctypes.c_int, [_P, _I32, _I32, _I32, _P, _I32, _P, _I32, _P]),
    "dec_diag_rmsnorm": (ctypes.c_int, [_P, _P, _I32, _I32, ctypes.c_double, _P, _P]),
    "dec_diag_quantize_rows": (ctypes.c_int, [_P, ctypes.c_int64, _I32, _P, _P, _P, _P]),
    "dec_diag_gemv": (ctypes.c_int, [_P, _I32, _P, _I32, _P, _P]),
    "dec_diag_quantize_q4": (ctypes.c_int, [_P, ctypes.c_int64, _I32, _P, _P, _P, _P]),
    "dec_diag_gemv_q4": (ctypes.c_int, [_P, _I32, _P, _P, _I32, _P, _P]),
    "dec_diag_moe_route": (ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "decoder_debug_layer_limit": (ctypes.c_int, [_P, _I32]),
    "decoder_debug_read_x": (ctypes.c_int, [_P, _P, _I32]),
    "decoder_debug_stop_after_attention": (ctypes.c_int, [_P, _I32]),
    "decoder_debug_fuse_o_proj": (ctypes.c_int, [_P, _I32]),
    "decoder_debug_fuse_ffn": (ctypes.c_int, [_P, _I32]),
    "decoder_debug_read_routes": (ctypes.c_int, [_P, _P, _I32]),
    "decoder_stats_enable": (ctypes.c_int, [_P, _I32]),
    "decoder_stats_read": (ctypes.c_int, [_P, ctypes.POINTER(DecoderStats)]),
    "decoder_stats_mask": (ctypes.c_int, [_P, _I32]),
}


def lib():
    """Load libdecoder.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m decoder_only_transformer_step_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


class DecoderError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (code {code})")
        self.code = code


def _check(rc, handle=None, what=""):
    if rc != DEC_OK:
        L = lib()
        detail = L.decoder_last_error(handle).decode() if handle else ""
        raise DecoderError(rc, f"{what}: {L.decoder_strerror(rc).decode()}" + (f" [{detail}]" if detail else ""))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _i32_array(values):
    vals = [int(v) for v in values]
    return (ctypes.c_int32 * max(1, len(vals)))(*vals), len(vals)


def make_config(shape):
    """decoder_config_t from a synth.workloads.Shape-like object."""
    s = shape
    return DecoderConfig(
        hidden=s.hidden, n_layers=s.n_layers, n_heads=s.n_heads, n_kv_heads=s.n_kv_heads,
        head_dim=s.head_dim, ffn_inter=s.ffn_inter, n_experts=s.n_experts, top_k=s.top_k,
        expert_inter=s.expert_inter, shared_inter=s.shared_inter, shared_gate=int(s.shared_gate),
        norm_topk_prob=int(s.norm_topk_prob), vocab=s.vocab, qkv_bias=int(s.qkv_bias),
        rope_base=float(s.rope_base), rms_eps=float(s.rms_eps), max_seq=s.max_seq,
        max_chunk=s.max_chunk, max_batch=s.max_batch, sliding_window=getattr(s, "sliding_window", 0),
        attn_softcap=float(getattr(s, "attn_softcap", 0.0)), qk_norm=int(getattr(s, "qk_norm", False)),
        weight_quant=int(getattr(s, "weight_quant", 0)), kv_page_size=int(getattr(s, "kv_page_size", 0)),
        kv_pages=int(getattr(s, "kv_pages", 0)))


# ---------------------------------------------------- same-named functions --

def decoder_workspace_bytes(cfg):
    return lib().decoder_workspace_bytes(ctypes.byref(cfg))


def decoder_init(cfg, weights, workspace, stream):
    """weights: dict with device tensors 'embed', 'final_norm', 'lm_head' and
    'layers' (list of dicts keyed by LAYER_FIELDS).  Returns (handle, keepalive)."""
    layers = (DecoderLayerWeights * cfg.n_layers)()
    for l, lw in enumerate(weights["layers"]):
        for f in LAYER_FIELDS:
            t = lw.get(f)
            if t is not None:
                setattr(layers[l], f, t.data_ptr())
    w = DecoderWeights(embed=weights["embed"].data_ptr(), final_norm=weights["final_norm"].data_ptr(),
                       lm_head=weights["lm_head"].data_ptr(), layers=layers)
    h = ctypes.c_void_p()
    rc = lib().decoder_init(ctypes.byref(cfg), ctypes.byref(w), ctypes.c_void_p(workspace.data_ptr()),
                            workspace.numel() * workspace.element_size(), ctypes.c_void_p(stream),
                            ctypes.byref(h))
    _check(rc, None, "decoder_init")
    return h, (layers, w)


def prefill_chunk(handle, seq, ids, start_pos, logits_mode=1, logits=None, argmax=None):
    arr, n = _i32_array(ids)
    _check(lib().prefill_chunk(handle, seq, arr, n, start_pos, logits_mode, _ptr(logits), _ptr(argmax)),
           handle, "prefill_chunk")


def decode_step(handle, seqs, tokens=None, logits=None, argmax=None):
    sarr, b = _i32_array(seqs)
    tarr = _i32_array(tokens)[0] if tokens is not None else None
    _check(lib().decode_step(handle, b, sarr, tarr, _ptr(logits), _ptr(argmax)), handle, "decode_step")


def kv_reset(handle, seq=-1):
    _check(lib().kv_reset(handle, seq), handle, "kv_reset")


def decode_run(handle, seq, n_steps, tokens):
    _check(lib().decode_run(handle, seq, n_steps, _ptr(tokens)), handle, "decode_run")


def kv_truncate(handle, seq, length):
    _check(lib().kv_truncate(handle, seq, length), handle, "kv_truncate")


def kv_load(handle, seq, layer, k, v, length):
    _check(lib().kv_load(handle, seq, layer, _ptr(k), _ptr(v), length), handle, "kv_load")


def decoder_seq_len(handle, seq):
    return lib().decoder_seq_len(handle, seq)


def decoder_free(handle):
    lib().decoder_free(handle)


# ------------------------------------------------------------- convenience --

class Decoder:
    """Owns the workspace tensor and the handle; methods mirror the C ABI."""

    def __init__(self, shape, weights, stream=None, device="cuda"):
        import torch
        self.shape = shape
        self.cfg = make_config(shape)
        nbytes = decoder_workspace_bytes(self.cfg)
        if nbytes == 0:
            raise DecoderError(DEC_E_INVALID, "invalid decoder config")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        self.weights = weights
        self.handle, self._keep = decoder_init(self.cfg, weights, self.workspace, self.stream.cuda_stream)

    def close(self):
        if getattr(self, "handle", None):
            decoder_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def prefill_chunk(self, seq, ids, start_pos, logits_mode=1, logits=None, argmax=None):
        prefill_chunk(self.handle, seq, ids, start_pos, logits_mode, logits, argmax)

    def decode_step(self, seqs, tokens=None, logits=None, argmax=None):
        decode_step(self.handle, seqs, tokens, logits, argmax)

    def kv_reset(self, seq=-1):
        kv_reset(self.handle, seq)

    def kv_truncate(self, seq, length):
        kv_truncate(self.handle, seq, length)

    def decode_run(self, seq, n_steps, tokens):
        decode_run(self.handle, seq, n_steps, tokens)

    def kv_load(self, seq, layer, k, v, length):
        kv_load(self.handle, seq, layer, k, v, length)

    def seq_len(self, seq=0):
        return decoder_seq_len(self.handle, seq)

    def set_stream(self, stream):
        """Launch later calls on `stream` (a torch.cuda.Stream); the library
        first waits for the work on the old one."""
        _check(lib().decoder_set_stream(self.handle, ctypes.c_void_p(stream.cuda_stream)), self.handle, "set_stream")
        self.stream = stream

    def debug_layer_limit(self, layers):
        _check(lib().decoder_debug_layer_limit(self.handle, layers), self.handle, "layer_limit")

    def debug_stop_after_attention(self, on):
        _check(lib().decoder_debug_stop_after_attention(self.handle, int(on)), self.handle, "stop_after_attention")

    def debug_fuse_o_proj(self, on):
        _check(lib().decoder_debug_fuse_o_proj(self.handle, int(on)), self.handle, "fuse_o_proj")

    def debug_fuse_ffn(self, on):
        _check(lib().decoder_debug_fuse_ffn(self.handle, int(on)), self.handle, "fuse_ffn")

    def debug_read_x(self, out, rows):
        _check(lib().decoder_debug_read_x(self.handle, _ptr(out), rows), self.handle, "read_x")

    def stats_enable(self, nodes=None):
        """nodes: iterable of node names to time (None: all), or () / False to stop."""
        if nodes is None or nodes is True:
            mask = -1
        elif not nodes:
            mask = 0
        else:
            mask = 0
            for n in nodes:
                mask |= 1 << NODES.index(n)
        _check(lib().decoder_stats_enable(self.handle, mask), self.handle, "stats_enable")

    def stats_mask(self, nodes):
        """Time only `nodes` from now on (no clearing, no wait)."""
        mask = 0
        for n in nodes:
            mask |= 1 << NODES.index(n)
        _check(lib().decoder_stats_mask(self.handle, mask), self.handle, "stats_mask")

    def stats_read(self):
        st = DecoderStats()
        _check(lib().decoder_stats_read(self.handle, ctypes.byref(st)), self.handle, "stats_read")
        return st.as_dict()

    def debug_read_routes(self, out, rows):
        _check(lib().decoder_debug_read_routes(self.handle, _ptr(out), rows), self.handle, "read_routes")


def diag_gemm(A, W, C, stream):
    M, K = A.shape
    N = W.shape[0]
    _check(lib().dec_diag_gemm(_ptr(A), M, K, _ptr(W), N, _ptr(C), ctypes.c_void_p(stream)), None, "dec_diag_gemm")


def diag_pack_w32(W, P, stream):
    """W bf16 [rows][K] -> P (same size): 32-row x 16-k MFMA tiles."""
    rows, K = W.shape
    _check(lib().dec_diag_pack_w32(_ptr(W), rows, K, _ptr(P), ctypes.c_void_p(stream)), None, "dec_diag_pack_w32")


def diag_gemm_chunk(A, Wp, C, ksplit, part, stream):
    """A: bf16 [planes][M][K] (planes 1 or 2), Wp: W [N][K] packed by
    diag_pack_w32, C fp32 [M][N]; part: fp32 scratch for the split partials
    (or None when ksplit == 1)."""
    planes, M, K = A.shape
    N = Wp.shape[0]
    n_part = part.numel() if part is not None else 0
    _check(lib().dec_diag_gemm_chunk(_ptr(A), planes, M, K, _ptr(Wp), N, _ptr(C), ksplit,
                                     _ptr(part) if part is not None else None, n_part,
                                     ctypes.c_void_p(stream)), None, "dec_diag_gemm_chunk")


def diag_gemm_grouped(A, Wp, E, a_rows, groups, C, stream):
    """A: bf16 [planes][M][K]; Wp: the stacked expert weights [E * N][K]
    packed by diag_pack_w32; a_rows int32 [P]; groups int32 [1 + 3 E]
    (count, expert[E], start[E], count[E]); C fp32 [P][N]."""
    planes, M, K = A.shape
    N = Wp.shape[0] // E
    P = a_rows.numel()
    _check(lib().dec_diag_gemm_grouped(_ptr(A), planes, M, K, _ptr(Wp), E, N, _ptr(a_rows), P, _ptr(groups),
                                       _ptr(C), ctypes.c_void_p(stream)),
           None, "dec_diag_gemm_grouped")


def diag_gemm_chunk_noalloc(A, Wp, C, ksplit, stream):
    """diag_gemm_chunk with the split partials in the library's static
    per-device array (no workspace, no allocation)."""
    planes, M, K = A.shape
    N = Wp.shape[0]
    _check(lib().dec_diag_gemm_chunk_noalloc(_ptr(A), planes, M, K, _ptr(Wp), N, _ptr(C), ksplit,
                                             ctypes.c_void_p(stream)), None, "dec_diag_gemm_chunk_noalloc")


def diag_quantize_q4(W, codes, exps, deq, stream):
    """W bf16 [rows][K] -> codes uint8 [rows][K / 2], exps int8 [rows][K / 32], deq bf16 [rows][K]."""
    rows, K = W.shape
    _check(lib().dec_diag_quantize_q4(_ptr(W), rows, K, _ptr(codes), _ptr(exps), _ptr(deq),
                                      ctypes.c_void_p(stream)), None, "dec_diag_quantize_q4")


def diag_gemv_q4(a, codes, exps, y, stream):
    N = codes.shape[0]
    K = a.shape[0]
    _check(lib().dec_diag_gemv_q4(_ptr(a), K, _ptr(codes), _ptr(exps), N, _ptr(y), ctypes.c_void_p(stream)),
           None, "dec_diag_gemv_q4")


def diag_gemv(a, W, y, stream):
    N, K = W.shape
    _check(lib().dec_diag_gemv(_ptr(a), K, _ptr(W), N, _ptr(y), ctypes.c_void_p(stream)), None, "dec_diag_gemv")


def diag_moe_route(logits, k, renorm, ids, wts, stream):
    rows, E = logits.shape
    _check(lib().dec_diag_moe_route(_ptr(logits), rows, E, k, int(renorm), _ptr(ids), _ptr(wts),
                                    ctypes.c_void_p(stream)), None, "dec_diag_moe_route")


def diag_quantize_rows(W, rows, K, q, scale, deq, stream=0):
    _check(lib().dec_diag_quantize_rows(_ptr(W), rows, K, _ptr(q), _ptr(scale), _ptr(deq), ctypes.c_void_p(stream)),
           None, "dec_diag_quantize_rows")


def diag_rmsnorm(x, g, eps, out, stream):
    rows, H = x.shape
    _check(lib().dec_diag_rmsnorm(_ptr(x), _ptr(g), rows, H, float(eps), _ptr(out), ctypes.c_void_p(stream)),
           None, "dec_diag_rmsnorm")
