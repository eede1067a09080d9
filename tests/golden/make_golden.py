"""Writes the golden fixtures from closed forms (no library calls at all).

hand_case_h4.json -- one layer, one head (H = d = 4), W_q = W_k = 0,
W_v = W_o = I, zero FFN, unit gains, lm_head = I, embedding row 0 = (2,0,0,0).
Block order and RMSNorm form: engine.zig, Engine.forward and rmsnormColumn;
decoder.rs module doc.  With one cached key the softmax weight is 1, so the
attention output is v = a = x / sqrt(mean(x^2) + eps) = x / sqrt(1 + eps),
x1 = x + a, the FFN adds nothing, and the logits are
x1 / sqrt(mean(x1^2) + eps).
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def hand_case():
    eps = 1e-5
    c = 2.0 + 2.0 / math.sqrt(1.0 + eps)
    return {
        "cite": "engine.zig Engine.forward / rmsnormColumn; decoder.rs module doc (block order)",
        "derivation": "x=(2,0,0,0); a=x/sqrt(1+eps); x1=x+a; logits=x1/sqrt(mean(x1^2)+eps)",
        "rms_eps": eps,
        "embed_row0": [2.0, 0.0, 0.0, 0.0],
        "expected_logits": [c / math.sqrt(c * c / 4.0 + eps), 0.0, 0.0, 0.0],
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "hand_case_h4.json"), "w") as f:
        json.dump(hand_case(), f, indent=1)
        f.write("\n")
