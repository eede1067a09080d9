"""Exact check of the MoE expert choices on the GPU's own router input.

End to end, the router of layer l reads RMSNorm(x) of the residual x that
the GPU itself computed, which differs from the oracle's x by the model's
accumulated rounding; near-ties of the k-th expert then flip for a reason
that has nothing to do with the router.  So the choices are checked layer by
layer on identical input: the library stops a rerun of the same step after
layer l's attention sub-block (decoder_debug_stop_after_attention) and hands
back that x; the oracle normalises it, computes the router logits in fp64
and takes the top-k (pipeline.rs MoeFfn: softmax over every expert, the k
largest, lower index first on ties).  The ids, in router order, must equal
the GPU's at every (layer, token).  The only freedom left is the GPU's own
fp32 arithmetic of the same logits: an entry may differ only where the
oracle's logits of the two experts involved are within TIE of each other
(logged as a near-tie).  TIE = 1e-4 is ten times the largest error of the
GPU's router logits from the same x: the activation enters as split bf16
(about 2^-17 relative per element), the router rows are N(0, 1/sqrt(H)),
so the logit error is about 2^-17 |b| ~ 1e-5 (H = 2048), and the fp32
accumulation adds less.
"""
import numpy as np

import oracle
from tests.gpu_util import log

TIE = 1e-4


def forced(dec, shape, rows):
    """The GPU's expert ids of its last call ([L][rows][k]), for the oracle to
    follow (force_routes): the end-to-end comparison then runs both sides on
    the same expert sets, as a teacher-forced decode runs both on the same
    token; that those sets are the router's correct choice on the GPU's own
    input is what check_routes_exact shows."""
    return read_routes(dec, shape, rows)


def read_routes(dec, shape, rows):
    import torch
    got = torch.empty((shape.n_layers, rows, shape.top_k), dtype=torch.int32, device="cuda")
    dec.debug_read_routes(got, rows)
    torch.cuda.synchronize()
    return got.cpu().numpy()


def check_routes_exact(dec, shape, W, rows, rerun, what):
    """The last call (run by the caller with all layers) routed `rows` rows;
    `rerun()` repeats that call from the same cache state.  Returns the number
    of near-ties."""
    import torch
    got = read_routes(dec, shape, rows)
    H, E, k = shape.hidden, shape.n_experts, shape.top_k
    x = torch.empty((rows, H), dtype=torch.float32, device="cuda")
    ties = 0
    try:
        dec.debug_stop_after_attention(1)
        for l in range(shape.n_layers):
            dec.debug_layer_limit(l + 1)
            rerun()
            dec.debug_read_x(x, rows)
            torch.cuda.synchronize()
            xm = x.cpu().numpy().astype(np.float64)
            L = W["layers"][l]
            b = np.stack([oracle.rmsnorm(xm[i], L["ffn_norm"], shape.rms_eps) for i in range(rows)])
            r = oracle.matmul(L["w_router"], E, H, b)
            for i in range(rows):
                ids, _, _ = oracle.route(r[i], k, shape.norm_topk_prob)
                g = got[l, i]
                if np.array_equal(ids, g):
                    continue
                gaps = np.abs(r[i][ids] - r[i][g])
                log(what, f"near-tie at layer {l} row {i}: gpu {list(map(int, g))} oracle {list(map(int, ids))} "
                          f"logit gaps {np.array2string(gaps, precision=2)}")
                assert len(set(map(int, g))) == k, f"{what}: repeated expert at layer {l} row {i}"
                assert gaps.max() < TIE, f"{what}: expert ids differ at layer {l} row {i} (gap {gaps.max():.2e})"
                ties += 1
    finally:
        dec.debug_stop_after_attention(0)
        dec.debug_layer_limit(-1)
    rerun()           # back to the full-depth state of the call
    torch.cuda.synchronize()
    log(what, "routes exact on identical input;", ties, "near-ties of", shape.n_layers * rows)
    return ties
