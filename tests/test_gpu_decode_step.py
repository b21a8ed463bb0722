"""GPU parity of the one-launch decode step: the step's new K/V rows appended
at each sequence's last position inside the attention kernel, and split-K
partitions merged by the last workgroup of each row.

Bars: the step's output equals, bit for bit, reshape_and_cache with the
table's slots followed by the two-kernel decode (same partition size),
whether split rows are merged by the reduce kernel or inside the launch
(PKV_MERGE_IN_KERNEL); its cache equals theirs bit for bit (NaN in the
appended slots before the call), and both are within 2e-3 of the oracle;
with the in-launch merge the workspace counters are zero after every call,
so a workspace serves call after call.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_366_amd as pkv
from oracle import attention as A
from synth import workloads as W

from gpu_common import DEV, i32, out_f64, to_dev

pytestmark = pytest.mark.gpu

WAVE, MFMA, AUTO = pkv.PKV_ALGO_WAVE, pkv.PKV_ALGO_MFMA, pkv.PKV_ALGO_AUTO
IN = pkv.PKV_MERGE_IN_KERNEL
TOL16 = 2e-3


class StepCase:
    """A decode batch whose last position's K/V are held back as the step's
    new rows; the device pool holds NaN in those slots."""

    def __init__(self, seed, lens, hq, hkv, D, dtype, int8=False):
        self.c = c = W.decode_case(seed, len(lens), hq, hkv, D, lens=lens, dtype=dtype,
                                   int8=int8)
        self.dtype, self.int8 = dtype, int8
        bs = 16
        self.slots = np.array([c.block_tables[s][(n - 1) // bs] * bs + (n - 1) % bs if n else -1
                               for s, n in enumerate(c.context_lens)], np.int32)
        live = self.slots >= 0
        S, H = len(lens), hkv
        nk = np.zeros((S, H, D), np.float32)
        nv = np.zeros((S, H, D), np.float32)
        blk, row = self.slots[live] // bs, self.slots[live] % bs
        nk[live] = c.k_cache[blk, :, row, :]
        nv[live] = c.v_cache[blk, :, row, :]
        self.new_k, self.new_v = to_dev(nk, dtype), to_dev(nv, dtype)
        self.q = to_dev(c.q, dtype)
        self.tables, self.lens = i32(c.block_tables), i32(c.context_lens)
        self.max_ctx = int(max(int(c.context_lens.max()), 1))
        if int8:
            self.k0 = torch.from_numpy(c.k_i8).to(DEV)
            self.v0 = torch.from_numpy(c.v_i8).to(DEV)
            self.ks = torch.from_numpy(c.k_scale).to(DEV)
            self.vs = torch.from_numpy(c.v_scale).to(DEV)
        else:
            kc, vc = c.k_cache.copy(), c.v_cache.copy()
            kc[blk, :, row, :] = np.nan
            vc[blk, :, row, :] = np.nan
            self.k0, self.v0 = to_dev(kc, dtype), to_dev(vc, dtype)
            self.ks = self.vs = None

    def oracle(self):
        c = self.c
        if self.int8:
            return A.decode(c.q, c.k_i8, c.v_i8, c.block_tables, c.context_lens, c.scale,
                            k_scale=c.k_scale, v_scale=c.v_scale)
        return A.decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.scale)

    def two_kernels(self, parts, algo, out_dtype=torch.float32):
        k, v = self.k0.clone(), self.v0.clone()
        if not self.int8:
            pkv.pkv_reshape_and_cache(self.new_k, self.new_v, k, v, i32(self.slots))
        out = torch.empty(self.q.shape, dtype=out_dtype, device=DEV)
        pkv.pkv_paged_attention_decode(out, self.q, k, v, self.tables, self.lens, self.max_ctx,
                                       float(self.c.scale), parts, algo, self.ks, self.vs)
        torch.cuda.synchronize()
        return out, k, v

    def step(self, parts, algo, ws=None, out_dtype=torch.float32, append=True):
        k, v = self.k0.clone(), self.v0.clone()
        out = torch.empty(self.q.shape, dtype=out_dtype, device=DEV)
        nk, nv = (self.new_k, self.new_v) if append else (None, None)
        ws = pkv.pkv_paged_attention_decode_step(out, self.q, nk, nv, k, v, self.tables,
                                                 self.lens, self.max_ctx, float(self.c.scale),
                                                 parts, algo, self.ks, self.vs, workspace=ws)
        torch.cuda.synchronize()
        return out, k, v, ws


def same_bits(x, y):
    if x.dtype in (torch.bfloat16, torch.float16):
        return torch.equal(x.view(torch.int16), y.view(torch.int16))
    if x.dtype == torch.float32:
        return torch.equal(x.view(torch.int32), y.view(torch.int32))
    return torch.equal(x, y)


def counters_zero(ws, S, hq, D, max_ctx, parts):
    n = pkv.pkv_decode_workspace_bytes(S, hq, D, max_ctx, parts)
    return not ws[n:].any().item() if ws is not None else True


LENS = [1, 15, 16, 17, 100, 1023, 1024, 1025, 1536, 1537, 2048, 3000, 0, 33]


@pytest.mark.parametrize("kind", ["mha-bf16", "mha-f16", "mha-f32", "gqa-bf16", "gqa8-bf16"])
def test_step_equals_reshape_then_decode(kind):
    hq, hkv, D = {"mha": (8, 8, 128), "gqa": (16, 2, 128), "gqa8": (32, 4, 64)}[
        kind.split("-")[0]]
    dtype = kind.split("-")[1]
    sc = StepCase(700 + len(kind), LENS, hq, hkv, D, dtype)
    ref64 = sc.oracle()
    algos = [WAVE] + ([MFMA, AUTO] if dtype != "f32" and hq != hkv else [AUTO])
    for algo in algos:
        for parts in (0, 64, 256, 1024, 1536):
            o2, k2, v2 = sc.two_kernels(parts, algo)
            for merge in (0, IN):
                o1, k1, v1, ws = sc.step(parts, algo | merge)
                assert same_bits(o1, o2), (algo, parts, merge, (o1 - o2).abs().max().item())
                assert same_bits(k1, k2) and same_bits(v1, v2), (algo, parts, merge)
                assert np.abs(out_f64(o1) - ref64).max() <= (1e-5 if dtype == "f32" else TOL16)
                assert counters_zero(ws, len(LENS), hq, D, sc.max_ctx, parts)
                # the same workspace again: counters were left at zero
                o3, _, _, _ = sc.step(parts, algo | merge, ws=ws)
                assert same_bits(o3, o1)


@pytest.mark.parametrize("algo", [WAVE, MFMA], ids=["wave", "mfma"])
def test_step_merge_over_hundreds_of_partitions(algo):
    """Rows of up to 313 partitions (16-token partitions over 5,000 keys):
    the reduce holds the (max, sum) pairs of partitions 0..255 in lane
    registers and re-reads the rest, the in-launch merge reads them all in
    order, and both give the same bits."""
    sc = StepCase(760 + algo, [5000, 4112, 4097, 1100, 17, 1], 16, 2, 128, "bf16")
    ref64 = sc.oracle()
    for parts in (16, 32):
        o2, k2, v2 = sc.two_kernels(parts, algo)
        for merge in (0, IN):
            o1, k1, v1, ws = sc.step(parts, algo | merge)
            assert same_bits(o1, o2), (parts, merge, (o1 - o2).abs().max().item())
            assert same_bits(k1, k2) and same_bits(v1, v2), (parts, merge)
            assert np.abs(out_f64(o1) - ref64).max() <= TOL16
            assert counters_zero(ws, 6, 16, 128, sc.max_ctx, parts)


@pytest.mark.parametrize("group", [3, 5, 7, 12])
def test_step_group_sizes_not_powers_of_two(group):
    """The new row of a KV head is written once, by one of the workgroups
    that share it, whatever the group: the cache and the output equal the
    two-kernel path bit for bit."""
    sc = StepCase(770 + group, [1, 17, 300, 1500, 3001], 2 * group, 2, 128, "bf16")
    ref64 = sc.oracle()
    for algo in (WAVE, MFMA):
        for parts in (0, 256):
            o2, k2, v2 = sc.two_kernels(parts, algo)
            for merge in (0, IN):
                o1, k1, v1, _ = sc.step(parts, algo | merge)
                assert same_bits(o1, o2), (algo, parts, merge)
                assert same_bits(k1, k2) and same_bits(v1, v2), (algo, parts, merge)
                assert np.abs(out_f64(o1) - ref64).max() <= TOL16


def test_step_workspace_reused_by_a_smaller_batch_and_bf16_output():
    big = StepCase(731, [3000, 5, 2049, 4096, 700, 1600], 16, 2, 128, "bf16")
    small = StepCase(732, [1600, 40, 3100], 16, 2, 128, "bf16")
    ws = None
    for sc in (big, small, big):
        for algo in (WAVE, MFMA, WAVE | IN, MFMA | IN):
            o2, _, _ = sc.two_kernels(512, algo & ~IN)
            if ws is None:
                _, _, _, ws = sc.step(512, algo)
            o1, _, _, ws = sc.step(512, algo, ws=ws)
            assert same_bits(o1, o2)
            ob, _, _, ws = sc.step(512, algo, ws=ws, out_dtype=torch.bfloat16)
            assert same_bits(ob, o1.to(torch.bfloat16))


def test_step_without_append_merges_int8_in_kernel():
    sc = StepCase(733, [9000, 1, 513, 4097, 16], 16, 2, 128, "bf16", int8=True)
    ref64 = sc.oracle()
    for algo in (WAVE, MFMA):
        for parts in (0, 512):
            o2, _, _ = sc.two_kernels(parts, algo)
            for merge in (0, IN):
                o1, _, _, ws = sc.step(parts, algo | merge, append=False)
                assert same_bits(o1, o2), (algo, parts, merge)
                assert np.abs(out_f64(o1) - ref64).max() <= TOL16
                assert counters_zero(ws, 5, 16, 128, sc.max_ctx, parts)
    out = torch.empty(sc.q.shape, dtype=torch.float32, device=DEV)
    with pytest.raises(pkv.PkvError, match="quantise-on-write"):
        pkv.pkv_paged_attention_decode_step(out, sc.q, sc.new_k, sc.new_v, sc.k0, sc.v0,
                                            sc.tables, sc.lens, sc.max_ctx, float(sc.c.scale),
                                            512, MFMA, sc.ks, sc.vs)


@pytest.mark.slow
def test_step_at_7b_shape_sampled():
    """The 7B-shape batch in the launch shape the benchmark times (1,536-token
    partitions, 16-wave workgroups, streaming loads): the step equals
    reshape_and_cache + decode + reduce bit for bit, and sampled rows match
    the oracle."""
    c = W.llama7b_decode(seed=1)
    bs = 16
    slots = np.array([c.block_tables[s][(n - 1) // bs] * bs + (n - 1) % bs
                      for s, n in enumerate(c.context_lens)], np.int32)
    blk, row = slots // bs, slots % bs
    nk, nv = c.k_cache[blk, :, row, :].copy(), c.v_cache[blk, :, row, :].copy()
    kc, vc = c.k_cache.copy(), c.v_cache.copy()
    kc[blk, :, row, :] = np.nan
    vc[blk, :, row, :] = np.nan
    k0, v0 = to_dev(kc, "bf16"), to_dev(vc, "bf16")
    del kc, vc
    q, tables, lens = to_dev(c.q, "bf16"), i32(c.block_tables), i32(c.context_lens)
    mc = int(c.context_lens.max())
    new_k, new_v = to_dev(nk, "bf16"), to_dev(nv, "bf16")
    k, v = k0.clone(), v0.clone()
    pkv.pkv_reshape_and_cache(new_k, new_v, k, v, i32(slots))
    o2 = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    pkv.pkv_paged_attention_decode(o2, q, k, v, tables, lens, mc, float(c.scale), 1536, AUTO)
    del k, v
    o1 = torch.empty_like(o2)
    for merge in (IN, 0):   # the default (reduce kernel) last, for the sampled check
        k, v = k0.clone(), v0.clone()
        pkv.pkv_paged_attention_decode_step(o1, q, new_k, new_v, k, v, tables, lens, mc,
                                            float(c.scale), 1536, AUTO | merge)
        torch.cuda.synchronize()
        assert same_bits(o1, o2), merge
        del k, v
    # the 7B step the benchmark times: 2,048-token partitions (no split)
    o3 = torch.empty_like(o2)
    pkv.pkv_paged_attention_decode_step(o3, q, new_k, new_v, k0.clone(), v0.clone(), tables,
                                        lens, mc, float(c.scale), 2048, AUTO)
    torch.cuda.synchronize()
    assert (o3 - o2).abs().max().item() <= 1e-5
    got = o1.cpu().numpy()
    rng = np.random.default_rng(2)
    for s, h in zip(rng.integers(0, 64, 12), rng.integers(0, 32, 12)):
        n = int(c.context_lens[s])
        K = A.gather(c.k_cache, c.block_tables[s], n, bs)[:, h]
        V = A.gather(c.v_cache, c.block_tables[s], n, bs)[:, h]
        assert np.abs(got[s, h] - A.attend(c.q[s, h], K, V, c.scale)).max() <= TOL16
    del k0, v0
    torch.cuda.empty_cache()
