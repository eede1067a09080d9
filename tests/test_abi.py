"""The C-ABI library loads, exports every symbol the headers declare, and
validates configs on the host (no GPU needed)."""
import ctypes
import glob
import os
import re

import pytest

from decoder_only_transformer_step_amd import binding
from synth.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M):
            if not m.group(0).lstrip().startswith(("typedef", "#", "return")):
                names.add(m.group(1))
    return names


def test_headers_declare_the_boundary():
    names = declared_functions()
    for n in ("decoder_init", "prefill_chunk", "decode_step", "kv_reset", "decoder_workspace_bytes",
              "decoder_free", "kv_load", "kv_truncate", "dec_diag_gemm"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(binding.LIB_PATH)
    missing = [n for n in sorted(declared_functions()) if not hasattr(L, n)]
    assert not missing, missing
    assert set(binding.SIGNATURES) == declared_functions()


def test_strerror_and_workspace_sizes():
    L = binding.lib()
    assert L.decoder_strerror(0) == b"ok"
    assert b"overflow" in L.decoder_strerror(1)
    for key, (shape, work) in WORKLOADS.items():
        cfg = binding.make_config(shape)
        nb = binding.decoder_workspace_bytes(cfg)
        assert nb > 0, key
        kv = 2 * shape.max_batch * shape.n_layers * shape.n_kv_heads * ((shape.max_seq + 31) // 32 * 32) \
            * shape.head_dim * 2
        assert nb >= kv
    assert WORKLOADS["longctx"][0].max_batch == 16


@pytest.mark.parametrize("field,value", [("n_kv_heads", 3), ("head_dim", 96), ("max_chunk", 0),
                                         ("hidden", 100), ("max_chunk", 1024), ("sliding_window", -1),
                                         ("attn_softcap", -1.0), ("qk_norm", 2), ("weight_quant", 2),
                                         ("kv_page_size", 48), ("kv_page_size", -32)])
def test_invalid_configs_rejected(field, value):
    shape = WORKLOADS["tiny"][0].with_(**{field: value})
    assert binding.decoder_workspace_bytes(binding.make_config(shape)) == 0


def test_init_rejects_missing_workspace():
    cfg = binding.make_config(WORKLOADS["tiny"][0])
    h = ctypes.c_void_p()
    w = binding.DecoderWeights()
    rc = binding.lib().decoder_init(ctypes.byref(cfg), ctypes.byref(w), None, 0, None, ctypes.byref(h))
    assert rc == binding.DEC_E_INVALID     # weights missing


def test_variant_configs_and_their_workspace():
    tiny = WORKLOADS["tiny"][0]
    base = binding.decoder_workspace_bytes(binding.make_config(tiny))
    # a paged cache needs its pages; with them its KV pool replaces the
    # per-sequence regions (4 pages of 32 positions vs 64 positions of 1 sequence)
    assert binding.decoder_workspace_bytes(binding.make_config(tiny.with_(kv_page_size=32))) == 0
    paged = binding.decoder_workspace_bytes(binding.make_config(tiny.with_(kv_page_size=32, kv_pages=4)))
    assert paged > 0
    # quantised weights add codes, scales and dequantised copies: 3 bytes per weight and more
    q8 = binding.decoder_workspace_bytes(binding.make_config(tiny.with_(weight_quant=1)))
    assert q8 - base >= 3 * (tiny.n_params() - tiny.vocab * tiny.hidden)
    # rows that are not a multiple of 16 cannot stream int8 codes
    assert binding.decoder_workspace_bytes(binding.make_config(tiny.with_(weight_quant=1, ffn_inter=680))) == 0
    moe = WORKLOADS["moe"][0]
    assert binding.decoder_workspace_bytes(binding.make_config(moe.with_(weight_quant=1))) > \
        binding.decoder_workspace_bytes(binding.make_config(moe))
    assert binding.decoder_workspace_bytes(binding.make_config(moe.with_(weight_quant=1, expert_inter=1400))) == 0
    for kw in (dict(sliding_window=8), dict(attn_softcap=30.0), dict(qk_norm=True)):
        assert binding.decoder_workspace_bytes(binding.make_config(tiny.with_(**kw))) == base


def test_attention_work_list_bounds():
    """Configs whose attention work lists cannot fit the split buffers (a
    decode batch of max_batch x n_kv_heads groups, or a prefill chunk's row
    groups x n_kv_heads) are refused up front instead of failing at a step."""
    tiny = WORKLOADS["tiny"][0]
    wide = tiny.with_(n_heads=64, n_kv_heads=64, head_dim=64)
    assert binding.decoder_workspace_bytes(binding.make_config(wide.with_(max_batch=128))) > 0   # 8192 groups
    assert binding.decoder_workspace_bytes(binding.make_config(wide.with_(max_batch=129))) == 0
