"""Marshalling helpers: storage-format arrays (host numpy) -> library descriptors and device tensors.

Nothing here computes: it maps type names to the C enums, copies arrays to the GPU with
the dtype views the kernels expect, and allocates outputs.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (A_BF16, A_F16, A_FP4_E2M1, A_FP8_E4M3, C_NATIVE, C_W_TO_FP8, O_BF16, O_F16, S_BF16, S_F16, S_F32, S_UE8M0,
               W_FP4_E2M1, W_FP8_E4M3, W_INT4, W_UINT4, make_desc, prepare, prepared_bytes)

_W = {"int4": W_INT4, "uint4": W_UINT4, "e2m1": W_FP4_E2M1, "e4m3": W_FP8_E4M3}
_S = {"f16": S_F16, "bf16": S_BF16, "f32": S_F32, "ue8m0": S_UE8M0}
_A = {"f16": A_F16, "bf16": A_BF16, "e4m3": A_FP8_E4M3, "e2m1": A_FP4_E2M1}
_O = {"f16": O_F16, "bf16": O_BF16}
_TORCH_OUT = {"f16": torch.float16, "bf16": torch.bfloat16}


def desc_for(layer, compute_flags: int = 0):
    return make_desc(_W[layer.w_type], _S[layer.s_type], layer.group, layer.z is not None, _A[layer.a_type],
                     (C_W_TO_FP8 if layer.compute == "w_to_fp8" else C_NATIVE) | compute_flags, _O[layer.out_type],
                     layer.experts, layer.n, layer.k)


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Copy a numpy array to the device keeping its bits (uint16/uint32 travel as int16/int32)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to(device)


def prepare_layer(layer, device="cuda", stream=None, compute_flags: int = 0):
    """Upload the logical tensors, run qg_prepare, return (handle, prepared buffer).

    compute_flags are OR-ed into the compute option (e.g. C_BATCH_INVARIANT).  The logical
    tensors are released after the stream has passed the transform.
    """
    desc = desc_for(layer, compute_flags)
    nbytes = prepared_bytes(desc)
    if nbytes == 0:
        raise ValueError(f"unsupported layer {layer.name}")
    buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
    w = to_dev(layer.w, device)
    s = to_dev(layer.s, device)
    z = None if layer.z is None else to_dev(layer.z, device)
    p = prepare(desc, w, s, z, buf, stream)
    torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()
    del w, s, z
    return p, buf


def acts_to_dev(acts, device="cuda"):
    x = to_dev(acts.x, device)
    xs = None if acts.x_scale is None else torch.from_numpy(np.ascontiguousarray(acts.x_scale)).to(device)
    return x, xs


def out_dtype(layer):
    return _TORCH_OUT[layer.out_type]


def out_bits_to_f64(y: torch.Tensor) -> np.ndarray:
    return y.float().cpu().numpy().astype(np.float64)
