"""MI355X-native decoder-only GQA transformer step (decode + chunked prefill).

The compute lives in libdecoder.so (hand-written HIP for gfx950, C ABI in
include/decoder.h); this package is its thin Python binding.
"""
from .binding import (Decoder, DecoderConfig, DecoderError, decode_step, decoder_free, decoder_init,
                      decoder_seq_len, decoder_workspace_bytes, kv_load, kv_reset, kv_truncate, lib,
                      make_config, prefill_chunk)

__all__ = ["Decoder", "DecoderConfig", "DecoderError", "decode_step", "decoder_free", "decoder_init",
           "decoder_seq_len", "decoder_workspace_bytes", "kv_load", "kv_reset", "kv_truncate", "lib",
           "make_config",
           "prefill_chunk"]
