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
                                         ("hidden", 100), ("max_chunk", 512)])
def test_invalid_configs_rejected(field, value):
    shape = WORKLOADS["tiny"][0].with_(**{field: value})
    assert binding.decoder_workspace_bytes(binding.make_config(shape)) == 0


def test_init_rejects_missing_workspace():
    cfg = binding.make_config(WORKLOADS["tiny"][0])
    h = ctypes.c_void_p()
    w = binding.DecoderWeights()
    rc = binding.lib().decoder_init(ctypes.byref(cfg), ctypes.byref(w), None, 0, None, ctypes.byref(h))
    assert rc == binding.DEC_E_INVALID     # weights missing
