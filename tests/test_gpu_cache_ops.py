"""GPU parity of reshape_and_cache and copy_blocks: bit-exact against the
oracle, every untouched slot or block unchanged (NaN patterns included)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_366_amd as pkv
from oracle import cache_ops as C
from synth import workloads as W

from gpu_common import DEV, i32, to_dev

pytestmark = pytest.mark.gpu


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    return t.numpy()


def host_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, np.float32).view(np.int32)
    if dtype == "f16":
        return np.ascontiguousarray(x, np.float32).astype(np.float16).view(np.int16)
    return W.storage_array(x, "bf16").view(np.int16)


@pytest.mark.parametrize("dtype,hkv,d,T", [("bf16", 32, 128, 2096), ("f32", 8, 64, 37),
                                            ("f16", 4, 128, 1), ("bf16", 8, 64, 300)])
def test_reshape_and_cache_bit_exact(dtype, hkv, d, T):
    rng = np.random.default_rng(T)
    nb = max(8, (T // 16) * 2)
    kc = W.draw_normal(rng, (nb, hkv, 16, d), dtype)
    vc = W.draw_normal(rng, (nb, hkv, 16, d), dtype)
    kc[rng.random(nb) < 0.3] = np.nan
    key = W.draw_normal(rng, (T, hkv, d), dtype)
    val = W.draw_normal(rng, (T, hkv, d), dtype)
    slots = W.distinct_slots(rng, nb * 16, T, skip_fraction=0.1)
    rk, rv = C.reshape_and_cache(key, val, kc, vc, slots, 16)
    dk, dv = to_dev(kc, dtype), to_dev(vc, dtype)
    pkv.pkv_reshape_and_cache(to_dev(key, dtype), to_dev(val, dtype), dk, dv, i32(slots))
    torch.cuda.synchronize()
    assert np.array_equal(bits(dk), host_bits(rk, dtype))
    assert np.array_equal(bits(dv), host_bits(rv, dtype))


def test_reshape_and_cache_reads_strided_rows():
    """key/value as views into a wider per-token row (e.g. a fused qkv tensor)."""
    rng = np.random.default_rng(5)
    T, hkv, d, nb = 40, 4, 64, 16
    qkv = W.draw_normal(rng, (T, 3, hkv, d), "bf16")
    kc = np.full((nb, hkv, 16, d), np.nan, np.float32)
    vc = kc.copy()
    slots = W.distinct_slots(rng, nb * 16, T)
    rk, rv = C.reshape_and_cache(qkv[:, 1], qkv[:, 2], kc, vc, slots, 16)
    dqkv = to_dev(qkv, "bf16")
    dk, dv = to_dev(kc, "bf16"), to_dev(vc, "bf16")
    pkv.pkv_reshape_and_cache(dqkv[:, 1], dqkv[:, 2], dk, dv, i32(slots))
    torch.cuda.synchronize()
    assert np.array_equal(bits(dk), host_bits(rk, "bf16"))
    assert np.array_equal(bits(dv), host_bits(rv, "bf16"))


@pytest.mark.parametrize("dtype", ["bf16", "f32", "i8"])
def test_copy_blocks_bit_exact(dtype):
    rng = np.random.default_rng(9)
    nb, hkv, d = 40, 32 if dtype == "bf16" else 8, 128 if dtype != "f32" else 64
    pairs = np.array([(1, 7), (1, 8), (4, 2), (30, 39), (12, 0)], np.int32)
    if dtype == "i8":
        kc = rng.integers(-128, 128, (nb, hkv, 16, d)).astype(np.int8)
        vc = rng.integers(-128, 128, (nb, hkv, 16, d)).astype(np.int8)
        ks = rng.random((nb, hkv)).astype(np.float32)
        vs = rng.random((nb, hkv)).astype(np.float32)
        rk, rv, rks, rvs = C.copy_blocks(kc, vc, pairs, ks, vs)
        dk, dv = torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV)
        dks, dvs = torch.from_numpy(ks).to(DEV), torch.from_numpy(vs).to(DEV)
        pkv.pkv_copy_blocks(dk, dv, i32(pairs), dks, dvs)
        torch.cuda.synchronize()
        assert np.array_equal(dk.cpu().numpy(), rk) and np.array_equal(dv.cpu().numpy(), rv)
        assert np.array_equal(dks.cpu().numpy(), rks) and np.array_equal(dvs.cpu().numpy(), rvs)
        return
    kc = W.draw_normal(rng, (nb, hkv, 16, d), dtype)
    vc = W.draw_normal(rng, (nb, hkv, 16, d), dtype)
    kc[3] = np.nan
    rk, rv, _, _ = C.copy_blocks(kc, vc, pairs)
    dk, dv = to_dev(kc, dtype), to_dev(vc, dtype)
    pkv.pkv_copy_blocks(dk, dv, i32(pairs))
    torch.cuda.synchronize()
    assert np.array_equal(bits(dk), host_bits(rk, dtype))
    assert np.array_equal(bits(dv), host_bits(rv, dtype))


def test_validation_rejects_unsafe_index_arrays(monkeypatch):
    monkeypatch.setenv("PKV_VALIDATE", "1")
    dk = torch.zeros((4, 2, 16, 64), dtype=torch.bfloat16, device=DEV)
    dv = torch.zeros_like(dk)
    key = torch.zeros((3, 2, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(pkv.PkvError):
        pkv.pkv_reshape_and_cache(key, key, dk, dv, i32([5, 9, 5]))       # duplicate slot
    with pytest.raises(pkv.PkvError):
        pkv.pkv_reshape_and_cache(key, key, dk, dv, i32([5, 9, 64]))      # outside the pool
    with pytest.raises(pkv.PkvError):
        pkv.pkv_copy_blocks(dk, dv, i32([[0, 1], [1, 2]]))                 # dst is a source
    with pytest.raises(pkv.PkvError):
        pkv.pkv_copy_blocks(dk, dv, i32([[0, 1], [2, 1]]))                 # dst twice
    with pytest.raises(pkv.PkvError):
        pkv.pkv_copy_blocks(dk, dv, i32([[0, 4]]))                         # outside the pool
