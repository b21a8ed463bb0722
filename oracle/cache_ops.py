"""Cache writes and block copies, as their plain definitions.

* ``reshape_and_cache``: only the new token's K/V is computed and appended to
  the cache each step ([nxbn] section 一); the per-token physical address is
  recorded by the page table ([nxbn] §2.2).  Here row t of the new keys and
  values goes to block ``slot // block_size``, row ``slot % block_size``, for
  every head; a negative slot means "skip this row".
* ``copy_blocks``: the data copy of copy-on-write — a new block receives the
  contents of the shared one before the writer appends ([kongchang] section
  "KV Cache内存共享").  Each (src, dst) pair copies K, V and, for int8
  storage, the per-block scales.
* ``swap_blocks``: preemption by swapping moves a preempted request's KV
  blocks from GPU memory to CPU memory and back when it resumes
  ([kongchang] section "抢占与恢复机制"; cold pages go to host memory in
  [cnnetsun] §2.3).  Each (src, dst) pair copies block src of one pool to
  block dst of another pool (K, V and, for int8 storage, the scales).

Both return new arrays and leave the inputs untouched.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np


def reshape_and_cache(key: np.ndarray, value: np.ndarray, k_cache: np.ndarray,
                      v_cache: np.ndarray, slot_mapping: Sequence[int],
                      block_size: int) -> Tuple[np.ndarray, np.ndarray]:
    kc = k_cache.copy()
    vc = v_cache.copy()
    for t, slot in enumerate(slot_mapping):
        slot = int(slot)
        if slot < 0:
            continue
        kc[slot // block_size, :, slot % block_size, :] = key[t]
        vc[slot // block_size, :, slot % block_size, :] = value[t]
    return kc, vc


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, pairs: Sequence[Tuple[int, int]],
                k_scale: Optional[np.ndarray] = None, v_scale: Optional[np.ndarray] = None):
    kc = k_cache.copy()
    vc = v_cache.copy()
    ks = None if k_scale is None else k_scale.copy()
    vs = None if v_scale is None else v_scale.copy()
    for src, dst in pairs:
        kc[int(dst)] = k_cache[int(src)]
        vc[int(dst)] = v_cache[int(src)]
        if ks is not None:
            ks[int(dst)] = k_scale[int(src)]
        if vs is not None:
            vs[int(dst)] = v_scale[int(src)]
    return kc, vc, ks, vs


def swap_blocks(dst_k: np.ndarray, dst_v: np.ndarray, src_k: np.ndarray, src_v: np.ndarray,
                pairs: Sequence[Tuple[int, int]], dst_ks: Optional[np.ndarray] = None,
                dst_vs: Optional[np.ndarray] = None, src_ks: Optional[np.ndarray] = None,
                src_vs: Optional[np.ndarray] = None):
    """Copies of the destination pools with ``dst[d] = src[s]`` for every
    (s, d) pair; every other destination block keeps its contents."""
    dk, dv = dst_k.copy(), dst_v.copy()
    dks = None if dst_ks is None else dst_ks.copy()
    dvs = None if dst_vs is None else dst_vs.copy()
    for s, d in pairs:
        dk[int(d)] = src_k[int(s)]
        dv[int(d)] = src_v[int(s)]
        if dks is not None:
            dks[int(d)] = src_ks[int(s)]
            dvs[int(d)] = src_vs[int(s)]
    return dk, dv, dks, dvs
