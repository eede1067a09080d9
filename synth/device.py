"""Synthetic inputs as torch device tensors: upload host-generated weights
(bit-identical to what the oracle reads) or generate them on the device with
the same generator definition (libsynth_dev.so) when they are too large to
build on the host quickly."""
import ctypes
import os

import numpy as np

from .weights import kv_seed, seed_of, tensor_specs

_HERE = os.path.dirname(os.path.abspath(__file__))
_DEV = None


def dev_lib():
    global _DEV
    if _DEV is None:
        path = os.path.join(_HERE, "libsynth_dev.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run `python synth/build.py`")
        L = ctypes.CDLL(path)
        L.synth_dev_normal_bf16.restype = ctypes.c_int
        L.synth_dev_normal_bf16.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                            ctypes.c_double, ctypes.c_uint64, ctypes.c_void_p]
        _DEV = L
    return _DEV


def dev_normal_bf16(t, seed, sigma, offset=0, stream=None):
    """Fill the bf16 tensor t with sigma * N(0,1) elements offset .. offset + numel - 1."""
    import torch
    st = stream if stream is not None else torch.cuda.current_stream()
    rc = dev_lib().synth_dev_normal_bf16(ctypes.c_void_p(t.data_ptr()), t.numel(), seed, float(sigma),
                                         offset, ctypes.c_void_p(st.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"synth_dev_normal_bf16 failed ({rc})")
    return t


def to_device(arr, device="cuda"):
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def upload_weights(host, device="cuda"):
    out = {"layers": []}
    for k in ("embed", "final_norm"):
        out[k] = to_device(host[k], device)
    out["lm_head"] = out["embed"] if host["lm_head"] is host["embed"] else to_device(host["lm_head"], device)
    for L in host["layers"]:
        out["layers"].append({k: to_device(v, device) for k, v in L.items()})
    return out


def device_weights(shape, device="cuda"):
    """Same tensors as synth.weights.host_weights, generated on the device."""
    import torch
    out = {"layers": [dict() for _ in range(shape.n_layers)]}
    for name, layer, numel, sigma, kind in tensor_specs(shape):
        if kind == "ones":
            t = torch.ones(numel, dtype=torch.float32, device=device)
        else:
            t = torch.empty(numel, dtype=torch.bfloat16, device=device)
            dev_normal_bf16(t, seed_of(name, layer), sigma)
            if kind == "f32":
                t = t.float()
            elif kind == "gain":
                t = t.float() + 1.0
        if layer is None:
            out[name] = t
        else:
            out["layers"][layer][name] = t
    if shape.tied:
        out["lm_head"] = out["embed"]
    return out


def device_kv(shape, seq, layer, length, device="cuda", out=None):
    """(K, V) bf16 [Hkv][length][d] fill for one (sequence, layer), N(0,1)."""
    import torch
    n = shape.n_kv_heads * length * shape.head_dim
    if out is None:
        out = (torch.empty(n, dtype=torch.bfloat16, device=device),
               torch.empty(n, dtype=torch.bfloat16, device=device))
    dev_normal_bf16(out[0][:n], kv_seed(seq, layer, 0), 1.0)
    dev_normal_bf16(out[1][:n], kv_seed(seq, layer, 1), 1.0)
    return out
