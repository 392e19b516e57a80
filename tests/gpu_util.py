"""Shared helpers for the GPU tests: move generated words to the device, run
the library through its Python binding, and compare with the oracle."""
import math

import numpy as np

TOL_O = {"fp16": 2e-3, "bf16": 1.6e-2}
TOL_LSE = 1e-4  # |dLSE| <= 1e-4 * max(1, |LSE_ref|)


def torch_dtype(dtype):
    import torch
    return {"fp16": torch.float16, "bf16": torch.bfloat16}[dtype]


def to_dev(words, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(words).view(np.int16).copy())
    return t.view(torch_dtype(dtype)).to("cuda:0")


def o_to_f64(o):
    return o.float().cpu().numpy().astype(np.float64)


def scale_for(D):
    return float(np.float32(1.0 / math.sqrt(D)))


def errors(o_gpu, lse_gpu, o_ref, lse_ref):
    """max |dO| and max |dLSE| / max(1, |LSE_ref|) over the given rows."""
    eo = float(np.abs(o_gpu - o_ref).max()) if o_ref.size else 0.0
    el = float((np.abs(lse_gpu - lse_ref) / np.maximum(1.0, np.abs(lse_ref))).max()) if lse_ref.size else 0.0
    return eo, el
