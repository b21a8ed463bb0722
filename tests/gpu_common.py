"""Helpers for the GPU parity tests: move synthetic host inputs to the device
in their storage dtype, and run the library's entry points on them."""
import numpy as np
import torch

import paged_kv_cache_366_amd as pkv
from synth import workloads as W

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
DEV = "cuda"


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Upload float32 values (exactly representable in ``dtype``)."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(x, np.float32).astype(np.float16)).to(DEV)
    if dtype == "bf16":
        bits = W.storage_array(x, "bf16").view(np.int16)
        return torch.from_numpy(bits).to(DEV).view(torch.bfloat16)
    raise ValueError(dtype)


def i32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(DEV)


class DevCase:
    """A PagedCase on the device."""

    def __init__(self, case: W.PagedCase, int8: bool = False):
        self.case = case
        self.dtype = case.dtype
        self.q = to_dev(case.q, case.dtype)
        if int8:
            self.k = torch.from_numpy(case.k_i8).to(DEV)
            self.v = torch.from_numpy(case.v_i8).to(DEV)
            self.ks = torch.from_numpy(case.k_scale).to(DEV)
            self.vs = torch.from_numpy(case.v_scale).to(DEV)
        else:
            self.k = to_dev(case.k_cache, case.dtype)
            self.v = to_dev(case.v_cache, case.dtype)
            self.ks = self.vs = None
        self.tables = i32(case.block_tables)
        self.lens = i32(case.context_lens)
        self.max_ctx = int(max(int(case.context_lens.max()), 1))

    def decode(self, parts=0, algo=pkv.PKV_ALGO_AUTO, out_dtype=torch.float32, lens=None,
               max_ctx=None, q=None):
        q = self.q if q is None else q
        out = torch.empty(q.shape, dtype=out_dtype, device=DEV)
        lens_t = self.lens if lens is None else lens
        mc = self.max_ctx if max_ctx is None else max_ctx
        pkv.pkv_paged_attention_decode(out, q, self.k, self.v, self.tables, lens_t, mc,
                                       float(self.case.scale), parts, algo, self.ks, self.vs)
        torch.cuda.synchronize()
        return out


def out_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def bf16_rne(x: torch.Tensor) -> torch.Tensor:
    """torch's float32 -> bfloat16 conversion (round to nearest even)."""
    return x.to(torch.bfloat16)
