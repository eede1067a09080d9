"""Helpers shared by the GPU parity tests: run the library and the oracle on
the same seeded inputs and compare with the acceptance rule
(logits max-abs <= 2e-2 and relative L2 <= 1e-2; greedy ids equal wherever
the oracle's top-2 margin exceeds 5e-2)."""
import sys

import numpy as np

MAX_ABS = 2e-2
REL_L2 = 1e-2
MARGIN = 5e-2


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def compare_logits(got, want, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite logits"
    err = np.abs(got - want)
    max_abs = float(err.max())
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    top2 = np.sort(want)[-2:]
    margin = float(top2[1] - top2[0])
    same = int(np.argmax(got)) == int(np.argmax(want))
    return dict(max_abs=max_abs, rel_l2=rel, margin=margin, argmax_same=same)


def assert_parity(stats, what=""):
    assert stats["max_abs"] <= MAX_ABS, f"{what}: max-abs {stats['max_abs']:.3e}"
    assert stats["rel_l2"] <= REL_L2, f"{what}: rel-L2 {stats['rel_l2']:.3e}"
    if stats["margin"] > MARGIN:
        assert stats["argmax_same"], f"{what}: greedy id differs at margin {stats['margin']:.3e}"


def make_decoder(shape, host_weights):
    import torch

    from decoder_only_transformer_step_amd import Decoder
    from synth.device import upload_weights
    dw = upload_weights(host_weights)
    dec = Decoder(shape, dw)
    torch.cuda.synchronize()
    return dec, dw


def run_prefill(dec, ids, chunk, seq=0, start=0):
    """Prefill ids in chunks; returns the last token's logits (numpy fp32)."""
    import torch
    logits = torch.empty(dec.shape.vocab, dtype=torch.float32, device="cuda")
    pos = start
    for c0 in range(0, len(ids), chunk):
        part = [int(t) for t in ids[c0:c0 + chunk]]
        dec.prefill_chunk(seq, part, pos, logits_mode=1, logits=logits)
        pos += len(part)
    torch.cuda.synchronize()
    return logits.cpu().numpy()


def decode(dec, seqs, tokens):
    """One decode step; returns ([B][V] logits, [B] argmax) as numpy."""
    import torch
    B = len(seqs)
    logits = torch.empty((B, dec.shape.vocab), dtype=torch.float32, device="cuda")
    am = torch.empty(B, dtype=torch.int32, device="cuda")
    dec.decode_step(seqs, tokens, logits=logits, argmax=am)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), am.cpu().numpy()
