"""Paged KV cache: the same model with a pool of fixed-size pages instead
of one contiguous region per sequence.

Paging changes where a (sequence, position) lives, never what is computed:
every kernel does the same arithmetic on the same values, so a paged
decoder's logits must equal a contiguous decoder's bit for bit, through
chunked prefill (chunks and key splits crossing pages), decode, ragged
batches, resets and rollbacks that hand pages from one sequence to another.
One run is also checked against the oracle.
"""
import numpy as np
import pytest

import oracle
from synth.weights import host_weights, prompt
from synth.workloads import C8B, TINY
from tests.gpu_util import assert_parity, compare_logits, decode, log, make_decoder, run_prefill

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SHAPES = {
    # (shape, page size, pages, prompt, chunk, decode steps)
    "tiny": (TINY, 32, 4, 40, 16, 6),
    "8b2": (C8B.with_(name="gqa-8b-layers-2", n_layers=2, vocab=1024, max_seq=512), 64, 6, 200, 128, 6),
}


def pair(which):
    shape, P, pages, _, _, _ = SHAPES[which]
    W = host_weights(shape)
    flat, _ = make_decoder(shape, W)
    paged, _ = make_decoder(shape.with_(kv_page_size=P, kv_pages=pages), W)
    return shape, W, flat, paged


@pytest.mark.parametrize("which", ["tiny", "8b2"])
def test_paged_equals_contiguous_bit_for_bit(which):
    _, _, _, Pr, chunk, steps = SHAPES[which]
    shape, W, flat, paged = pair(which)
    ids = prompt(shape, Pr)
    a = run_prefill(flat, ids, chunk)
    b = run_prefill(paged, ids, chunk)
    assert np.array_equal(a, b)
    want = oracle.Model(shape, W).prefill(ids, chunk)["logits"]
    assert_parity(compare_logits(b, want, f"{which} paged prefill"), f"{which} paged prefill")
    toks = prompt(shape, steps, seq=5)
    for i in range(steps):
        la, ia = decode(flat, [0], [int(toks[i])])
        lb, ib = decode(paged, [0], [int(toks[i])])
        assert np.array_equal(la, lb), f"decode {i}"
        assert np.array_equal(ia, ib)
    log(which, "paged == contiguous through", Pr, "prompt tokens and", steps, "decodes")
    flat.close()
    paged.close()


def test_paged_ragged_batch_reset_rollback_and_exhaustion():
    """Three sequences of different lengths share a pool of 4 pages of 32
    positions; a reset and a rollback return pages that other sequences then
    take (in a different order than a fresh pool hands them out)."""
    shape = TINY.with_(max_batch=3)
    W = host_weights(shape)
    flat, _ = make_decoder(shape, W)
    paged, _ = make_decoder(shape.with_(kv_page_size=32, kv_pages=4), W)
    both = (flat, paged)

    def prefill(seq, n, seed):
        ids = prompt(shape, n, seq=seed)
        out = [run_prefill(d, ids, 16, seq=seq, start=d.seq_len(seq)) for d in both]
        assert np.array_equal(out[0], out[1]), (seq, n)

    def step(seqs, seed):
        toks = [int(t) for t in prompt(shape, len(seqs), seq=seed)]
        out = [decode(d, seqs, toks) for d in both]
        assert np.array_equal(out[0][0], out[1][0]), seqs

    prefill(0, 40, 1)            # 2 pages
    prefill(1, 9, 2)             # 1 page
    prefill(2, 20, 3)            # 1 page: the pool is full
    step([0, 1, 2], 10)
    for k in range(3):           # growth inside the pages already held
        step([0, 2], 11 + k)
    # seq 2 at 24 + 16 positions needs a second page: refused, nothing changes
    with pytest.raises(Exception):
        paged.prefill_chunk(2, [1] * 16, paged.seq_len(2))
    assert paged.seq_len(2) == flat.seq_len(2) == 24
    # reset seq 0 (2 pages back), roll seq 2 back to 10 positions (keeps 1)
    for d in both:
        d.kv_reset(0)
        d.kv_truncate(2, 10)
    prefill(0, 16, 4)            # takes a returned page
    prefill(2, 16, 5)            # 26 positions: still its one page
    step([2, 0, 1], 20)
    prefill(1, 16, 6)            # 11 -> 27 positions
    prefill(1, 16, 7)            # 27 -> 43: takes the last free page
    step([1, 2], 21)
    log("ragged paged batch matches the contiguous decoder bit for bit")
    flat.close()
    paged.close()


def test_paged_with_every_option_and_verify():
    """Paging under int8 weights, a window, a soft-cap, sinks and QK-norm at
    once, through a verify of four drafts and a rollback: bit for bit the
    contiguous decoder, and within the acceptance rule of the oracle."""
    shape = C8B.with_(name="gqa-8b-layers-2-all", n_layers=2, vocab=1024, max_seq=512, weight_quant=1,
                      sliding_window=100, attn_softcap=2.0, attn_sinks=True, qk_norm=True)
    W = host_weights(shape)
    flat, _ = make_decoder(shape, W)
    paged, _ = make_decoder(shape.with_(kv_page_size=64, kv_pages=5), W)
    m = oracle.Model(shape, W)
    ids = prompt(shape, 150)
    a = run_prefill(flat, ids, 128)
    b = run_prefill(paged, ids, 128)
    assert np.array_equal(a, b)
    want = m.prefill(ids, 128)["logits"]
    assert_parity(compare_logits(b, want, "all options prefill"), "all options prefill")
    drafts = [int(t) for t in prompt(shape, 4, seq=9)]
    outs = []
    for d in (flat, paged):
        lg = torch.empty((4, shape.vocab), dtype=torch.float32, device="cuda")
        d.prefill_chunk(0, drafts, 150, logits_mode=2, logits=lg)
        torch.cuda.synchronize()
        outs.append(lg.cpu().numpy())
        d.kv_truncate(0, 152)
    assert np.array_equal(outs[0], outs[1])
    m.forward(drafts, 150, logits_mode=0)
    m.truncate(0, 152)
    nxt = int(prompt(shape, 1, seq=10)[0])
    la, _ = decode(flat, [0], [nxt])
    lb, _ = decode(paged, [0], [nxt])
    assert np.array_equal(la, lb)
    want = m.forward([nxt], 152)["logits"]
    assert_parity(compare_logits(lb[0], want, "all options decode after rollback"), "all options decode")
    flat.close()
    paged.close()


def test_paged_kv_load_equals_contiguous():
    """A KV prefix loaded into a paged cache (kv_load scatters K rows and V^T
    columns into the sequence's pages) decodes bit for bit like the same
    prefix loaded into the contiguous cache: three sequences of ragged
    lengths on the 8B-class layer shapes with pages of 64 positions, a
    reload to a shorter length that hands pages back, a pool too small for a
    further load (refused, nothing changed), then batched decode."""
    from synth.device import to_device
    from synth.weights import host_kv
    shape = C8B.with_(name="gqa-8b-layers-2-b3", n_layers=2, vocab=1024, max_seq=512, max_batch=3, max_chunk=16)
    W = host_weights(shape)
    P, pages = 64, 14
    flat, _ = make_decoder(shape, W)
    paged, _ = make_decoder(shape.with_(kv_page_size=P, kv_pages=pages), W)
    lens = [300, 130, 380]                       # 5 + 3 + 6 = 14 pages: the whole pool
    for s, n in enumerate(lens):
        for l in range(shape.n_layers):
            K, V = host_kv(shape, s, l, n)
            dk, dv = to_device(K), to_device(V)
            flat.kv_load(s, l, dk, dv, n)
            paged.kv_load(s, l, dk, dv, n)
    # reload seq 2 shorter: it keeps 3 of its 6 pages
    lens[2] = 190
    for l in range(shape.n_layers):
        K, V = host_kv(shape, 2, l, lens[2])
        dk, dv = to_device(K), to_device(V)
        flat.kv_load(2, l, dk, dv, lens[2])
        paged.kv_load(2, l, dk, dv, lens[2])
    assert [paged.seq_len(s) for s in range(3)] == lens
    # 5 + 3 + 3 = 11 pages in use: a load of seq 1 to 512 positions (8 pages) needs 5 more than the 3 left
    K, V = host_kv(shape, 1, 0, 512)
    with pytest.raises(Exception):
        paged.kv_load(1, 0, to_device(K), to_device(V), 512)
    assert paged.seq_len(1) == lens[1]
    toks = [int(t) for t in prompt(shape, 3, seq=17)]
    for step in range(3):
        a, am = decode(flat, [0, 1, 2], toks)
        b, _ = decode(paged, [0, 1, 2], toks)
        assert np.array_equal(a, b), f"step {step}"
        toks = [int(t) for t in am]
    log("paged kv_load equals the contiguous cache through 3 batched decode steps")
    flat.close()
    paged.close()
