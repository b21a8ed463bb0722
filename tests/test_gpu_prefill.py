"""GPU parity of chunked prefill attention against the float64 oracle.

Row i of a chunk of length q over a context of n tokens sits at position
n - q + i and attends keys [0, n - q + i] through the block table.  Bars as
for decode: max |gpu - oracle| <= 2e-3 for 16-bit inputs (fp32
accumulation), <= 1e-5 for fp32; bf16 output is the round-to-nearest-even of
the fp32 output bit for bit; physical placement never changes a bit.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_366_amd as pkv
from oracle import attention as A
from oracle import cache_ops as C
from synth import workloads as W

from gpu_common import DEV, i32, out_f64, to_dev

pytestmark = pytest.mark.gpu

TOL16 = 2e-3
TOL32 = 1e-5


def gpu_prefill(c, out_dtype=torch.float32, q=None, tables=None, kc=None, vc=None):
    qd = to_dev(c.q if q is None else q, c.dtype)
    k = to_dev(c.k_cache if kc is None else kc, c.dtype)
    v = to_dev(c.v_cache if vc is None else vc, c.dtype)
    t = i32(c.block_tables if tables is None else tables)
    qsl = c.query_start_loc
    out = torch.empty(qd.shape, dtype=out_dtype, device=DEV)
    max_q = int(np.diff(qsl).max())
    pkv.pkv_paged_attention_prefill(out, qd, k, v, t, i32(qsl), i32(c.context_lens), max_q,
                                    int(c.context_lens.max()), float(c.scale))
    torch.cuda.synchronize()
    return out


def oracle_prefill(c):
    return A.prefill(c.q, c.k_cache, c.v_cache, c.block_tables, c.query_start_loc,
                     c.context_lens, c.scale)


# (prior cached tokens, chunk length): ragged tails, exact blocks, chunks
# spanning several 64-row tiles, a one-row chunk and an empty one.
CHUNKS = [(0, 1), (0, 17), (7, 64), (16, 65), (100, 130), (33, 0), (250, 16), (5, 3)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("hq,hkv,d", [(4, 4, 128), (8, 2, 128), (4, 4, 64), (6, 3, 64),
                                      (10, 2, 128), (12, 4, 64)])
def test_prefill_matches_oracle(dtype, hq, hkv, d):
    c = W.prefill_case(500 + hq + d, hq, hkv, d, CHUNKS, dtype=dtype)
    ref = oracle_prefill(c)
    out = gpu_prefill(c)
    err = np.abs(out_f64(out) - ref).max()
    assert err <= TOL16, err
    assert err <= 1e-4, f"unexpectedly large error {err}"


def test_prefill_fp32_wavefront_path():
    c = W.prefill_case(77, 4, 2, 64, [(0, 9), (20, 40), (3, 1)], dtype="f32")
    err = np.abs(out_f64(gpu_prefill(c)) - oracle_prefill(c)).max()
    assert err <= TOL32, err


def test_prefill_bf16_output_is_rounded_fp32_output():
    c = W.prefill_case(78, 4, 4, 128, CHUNKS, dtype="bf16")
    of = gpu_prefill(c)
    ob = gpu_prefill(c, out_dtype=torch.bfloat16)
    assert torch.equal(ob.view(torch.int16), of.to(torch.bfloat16).view(torch.int16))


def test_prefill_placement_is_bit_invariant():
    c = W.prefill_case(79, 8, 2, 128, CHUNKS, dtype="bf16")
    base = gpu_prefill(c)
    perm = np.random.default_rng(5).permutation(c.num_blocks)
    kc = np.empty_like(c.k_cache)
    vc = np.empty_like(c.v_cache)
    kc[perm] = c.k_cache
    vc[perm] = c.v_cache
    tables = np.where(c.block_tables >= 0, perm[np.maximum(c.block_tables, 0)], -1)
    out = gpu_prefill(c, tables=tables.astype(np.int32), kc=kc, vc=vc)
    assert torch.equal(out, base)


def test_one_row_chunks_match_decode():
    # every sequence a chunk of one row: prefill must give the decode result
    c = W.prefill_case(80, 8, 8, 128, [(15, 1), (0, 1), (300, 1), (31, 1)], dtype="bf16")
    pre = out_f64(gpu_prefill(c))
    qd = to_dev(c.q, "bf16")
    out = torch.empty(qd.shape, dtype=torch.float32, device=DEV)
    pkv.pkv_paged_attention_decode(out, qd, to_dev(c.k_cache, "bf16"), to_dev(c.v_cache, "bf16"),
                                   i32(c.block_tables), i32(c.context_lens),
                                   int(c.context_lens.max()), float(c.scale), 0)
    torch.cuda.synchronize()
    ref = A.decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.scale)
    assert np.abs(pre - ref).max() <= TOL16
    assert np.abs(out_f64(out) - ref).max() <= TOL16


def test_large_scores_stay_finite():
    c = W.prefill_case(81, 4, 4, 128, [(40, 70)], dtype="bf16")
    q = W.round_bf16(c.q * np.float32(60))
    ref = A.prefill(q, c.k_cache, c.v_cache, c.block_tables, c.query_start_loc,
                    c.context_lens, c.scale)
    out = gpu_prefill(c, q=q)
    assert torch.isfinite(out).all()
    assert np.abs(out_f64(out) - ref).max() <= TOL16


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_stage_count_changes_no_bit(dtype):
    """At head_dim 128 a launch with more workgroups than compute units
    stages K/V in two LDS buffers, a smaller one in three.  The same chunk
    computed alone (a small grid) and as each of many identical sequences
    (a grid past the compute-unit count) gives the same bits."""
    hq = 8
    one = W.prefill_case(83, hq, 2, 128, [(300, 200)], dtype=dtype)
    tiles = -(-200 // 64)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = cus // (tiles * hq) + 2
    assert one.block_tables.shape[0] == 1 and n * tiles * hq > cus >= tiles * hq
    alone = gpu_prefill(one)
    qsl = np.arange(n + 1, dtype=np.int32) * 200
    qd = to_dev(np.concatenate([one.q] * n), dtype)
    out = torch.empty(qd.shape, dtype=torch.float32, device=DEV)
    pkv.pkv_paged_attention_prefill(out, qd, to_dev(one.k_cache, dtype), to_dev(one.v_cache, dtype),
                                    i32(np.repeat(one.block_tables, n, axis=0)), i32(qsl),
                                    i32(np.repeat(one.context_lens, n)), 200,
                                    int(one.context_lens.max()), float(one.scale))
    torch.cuda.synchronize()
    for r in range(n):
        assert torch.equal(out[200 * r:200 * (r + 1)], alone), r
    assert np.abs(out_f64(alone) - oracle_prefill(one)).max() <= TOL16


def test_batches_past_the_ranked_size():
    """Up to 256 sequences each workgroup ranks the batch by context length
    (longest first); a larger batch keeps index order.  Both orders give
    every row its own result: 300 short chunks against the oracle, and the
    first 200 of them alone (ranked) bit for bit against the same rows."""
    rng = np.random.default_rng(84)
    chunks = [(int(p), int(q)) for p, q in zip(rng.integers(0, 90, 300), rng.integers(1, 20, 300))]
    c = W.prefill_case(84, 4, 2, 128, chunks, dtype="bf16")
    out = gpu_prefill(c)
    assert np.abs(out_f64(out) - oracle_prefill(c)).max() <= TOL16
    n = 200
    rows = int(c.query_start_loc[n])
    part = W.prefill_case(84, 4, 2, 128, chunks[:n], dtype="bf16")
    sub = gpu_prefill(part, q=c.q[:rows], tables=c.block_tables[:n], kc=c.k_cache, vc=c.v_cache)
    # the same tables, pool and queries: only the batch size differs
    assert np.array_equal(part.query_start_loc, c.query_start_loc[:n + 1])
    assert torch.equal(sub, out[:rows])


def test_validation_rejects_a_chunk_longer_than_its_context(monkeypatch):
    c = W.prefill_case(82, 4, 4, 64, [(0, 10), (5, 5)], dtype="bf16")
    monkeypatch.setenv("PKV_VALIDATE", "1")
    lens = c.context_lens.copy()
    lens[0] = 9     # chunk of 10 rows over 9 tokens
    qd = to_dev(c.q, "bf16")
    out = torch.empty(qd.shape, dtype=torch.float32, device=DEV)
    with pytest.raises(pkv.PkvError):
        pkv.pkv_paged_attention_prefill(out, qd, to_dev(c.k_cache, "bf16"),
                                        to_dev(c.v_cache, "bf16"), i32(c.block_tables),
                                        i32(c.query_start_loc), i32(lens), 10, 10,
                                        float(c.scale))


# ---------------------------------------------------------------- mixed step
def run_mixed_step(ms, sample_rows=None, decode_parts=(256,)):
    """Allocate through the block manager, write every new row through
    reshape_and_cache, then run decode on the decode sequences (once per
    split-K partition size in `decode_parts`) and prefill on the chunks.
    The oracle side follows the same steps on host arrays."""
    nb, hkv, d = ms.num_blocks, ms.kv_heads, ms.head_dim
    bm = pkv.pkv_bm_create(nb, 16, ms.perm)
    try:
        kc = np.full((nb, hkv, 16, d), np.nan, np.float32)
        vc = kc.copy()
        dk, dv = to_dev(kc, ms.dtype), to_dev(vc, ms.dtype)
        seqs = []
        for s in range(len(ms.prior)):
            sid = pkv.pkv_seq_create(bm, int(ms.prior[s]))
            p = int(ms.prior[s])
            if p:
                # already-cached history: laid into the host image in place
                # (input preparation), written to the device pool by the library
                sl = pkv.pkv_seq_slots(bm, sid, 0, p)
                kc[sl // 16, :, sl % 16, :] = ms.prior_k[s]
                vc[sl // 16, :, sl % 16, :] = ms.prior_v[s]
                pkv.pkv_reshape_and_cache(to_dev(ms.prior_k[s], ms.dtype),
                                          to_dev(ms.prior_v[s], ms.dtype), dk, dv, i32(sl))
            seqs.append(sid)
        # the step: one slot mapping for every new token, one cache write
        slots = np.concatenate([pkv.pkv_seq_append(bm, sid, int(ms.new[s]))[0]
                                for s, sid in enumerate(seqs)])
        kc, vc = C.reshape_and_cache(ms.new_k, ms.new_v, kc, vc, slots, 16)
        pkv.pkv_reshape_and_cache(to_dev(ms.new_k, ms.dtype), to_dev(ms.new_v, ms.dtype), dk, dv,
                                  i32(slots))
        lens_all = ms.prior + ms.new
        mb = W.blocks_for(int(lens_all.max()))
        tables, lens = pkv.pkv_seq_export(bm, seqs, mb)
        assert np.array_equal(lens, lens_all)
        dec = np.flatnonzero(ms.new == 1)
        pre = np.flatnonzero(ms.new > 1)
        # token order: sequences in index order, decode sequences first
        starts = np.concatenate([[0], np.cumsum(ms.new)])
        qd_rows = starts[dec]
        qdev = to_dev(ms.q, ms.dtype)
        outs_d = []
        for part in decode_parts:
            out_d = torch.empty((len(dec),) + ms.q.shape[1:], dtype=torch.float32, device=DEV)
            pkv.pkv_paged_attention_decode(out_d,
                                           qdev[torch.from_numpy(qd_rows).to(DEV)].contiguous(),
                                           dk, dv, i32(tables[dec]), i32(lens[dec]),
                                           int(lens[dec].max()), float(ms.scale), part)
            outs_d.append(out_d)
        qsl = np.concatenate([[0], np.cumsum(ms.new[pre])]).astype(np.int32)
        rows = np.concatenate([np.arange(starts[s], starts[s + 1]) for s in pre])
        qp = qdev[torch.from_numpy(rows).to(DEV)].contiguous()
        out_p = torch.empty(qp.shape, dtype=torch.float32, device=DEV)
        pkv.pkv_paged_attention_prefill(out_p, qp, dk, dv, i32(tables[pre]), i32(qsl),
                                        i32(lens[pre]), int(ms.new[pre].max()),
                                        int(lens[pre].max()), float(ms.scale))
        torch.cuda.synchronize()
        # oracle
        ref_d = A.decode(ms.q[qd_rows], kc, vc, tables[dec], lens[dec], ms.scale)
        for part, out_d in zip(decode_parts, outs_d):
            assert np.abs(out_f64(out_d) - ref_d).max() <= TOL16, part
        got = out_f64(out_p)
        if sample_rows is None:
            ref_p = A.prefill(ms.q[rows], kc, vc, tables[pre], qsl, lens[pre], ms.scale)
            assert np.abs(got - ref_p).max() <= TOL16
        else:
            G = ms.q_heads // hkv
            rng = np.random.default_rng(0)
            for j, s in enumerate(pre):
                n, ql = int(lens[s]), int(ms.new[s])
                K = A.gather(kc, tables[s], n, 16)
                V = A.gather(vc, tables[s], n, 16)
                picks = set(rng.choice(ql, sample_rows, replace=False).tolist()) | {0, ql - 1}
                for i in sorted(picks):
                    P = n - ql + i
                    r = qsl[j] + i
                    for h in rng.choice(ms.q_heads, 4, replace=False):
                        ref = A.attend(ms.q[rows[r], h], K[:P + 1, h // G], V[:P + 1, h // G],
                                       ms.scale)
                        assert np.abs(got[r, h] - ref).max() <= TOL16, (s, i, h)
    finally:
        pkv.pkv_bm_destroy(bm)


def test_mixed_step_small():
    ms = W.mixed_step(seed=43, num_decode=6, decode_lens=(20, 300),
                      prefill_chunks=((0, 40), (24, 33), (100, 70)), q_heads=8, kv_heads=8,
                      head_dim=128)
    run_mixed_step(ms)


@pytest.mark.slow
def test_mixed_step_full_size_sampled():
    # 48 decode sequences (contexts U[64, 4096]) and four 512-row chunks over
    # 0/512/1024/1536 cached tokens, 32 heads x 128, bf16
    ms = W.mixed_step(seed=2)
    # the step's timed launch shape: the library's partition for these
    # decode lengths (one partition per context: the 1,536 workgroups need
    # several rounds unsplit); its 1.6 GB pool streams, so the wavefront
    # kernel runs 16-wave workgroups.  Plus a split at 256 tokens.
    dec = ms.new == 1
    timed = pkv.pkv_decode_partition_tokens(
        (ms.prior + ms.new)[dec], pkv.PKV_BF16, pkv.PKV_BF16, ms.q_heads, ms.kv_heads,
        ms.head_dim, W.BLOCK_SIZE, ms.num_blocks)
    assert timed == 0, timed
    run_mixed_step(ms, sample_rows=6, decode_parts=(256, timed))


# ------------------------------------------------------------ split-K prefill
LONG_CHUNKS = [(0, 70), (300, 130), (1000, 64), (777, 1), (33, 0), (64, 200), (1500, 17)]


def prefill_split(c, part, out_dtype=torch.float32, workspace=None):
    qd = to_dev(c.q, c.dtype)
    out = torch.empty(qd.shape, dtype=out_dtype, device=DEV)
    ws = pkv.pkv_paged_attention_prefill(
        out, qd, to_dev(c.k_cache, c.dtype), to_dev(c.v_cache, c.dtype), i32(c.block_tables),
        i32(c.query_start_loc), i32(c.context_lens), int(np.diff(c.query_start_loc).max()),
        int(c.context_lens.max()), float(c.scale), partition_tokens=part, workspace=workspace)
    torch.cuda.synchronize()
    return out, ws


def test_prefill_partition_choice():
    """Four 64-row chunks over 16,384 keys (128 workgroups unsplit) split so
    that two workgroups per compute unit are busy; the mixed step's chunks
    fill the GPU unsplit; fp32 q never splits; a chunk longer than its
    context is refused.  The chosen split of a small batch matches the
    oracle."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    p = pkv.pkv_prefill_partition_tokens([64] * 4, [16384] * 4, 32)
    n = lambda pt: 4 * 32 * -(-16384 // pt)
    assert p % 16 == 0 and p >= 256 and n(p) <= 2 * cus < n(p - 16), p
    assert pkv.pkv_prefill_partition_tokens([512] * 4, [512, 1024, 1536, 2048], 32) == 0
    assert pkv.pkv_prefill_partition_tokens([64] * 4, [16384] * 4, 32, pkv.PKV_F32) == 0
    with pytest.raises(pkv.PkvError):
        pkv.pkv_prefill_partition_tokens([65], [64], 32)
    c = W.prefill_case(95, 8, 2, 128, LONG_CHUNKS, dtype="bf16")
    p = pkv.pkv_prefill_partition_tokens(np.diff(c.query_start_loc), c.context_lens, 8)
    assert p >= 256, p
    out, _ = prefill_split(c, p)
    assert np.abs(out_f64(out) - oracle_prefill(c)).max() <= TOL16


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 8, 2, 128), ("f16", 4, 4, 64),
                                            ("f32", 4, 2, 64)])
def test_split_prefill_matches_oracle_and_unsplit(dtype, hq, hkv, d):
    c = W.prefill_case(90 + d, hq, hkv, d, LONG_CHUNKS, dtype=dtype)
    ref = oracle_prefill(c)
    base, ws0 = prefill_split(c, 0)
    assert ws0 is None
    tol = TOL32 if dtype == "f32" else TOL16
    for part in (16, 48, 256, 512):
        out, ws = prefill_split(c, part)
        assert ws is not None
        got = out_f64(out)
        assert np.abs(got - ref).max() <= tol, part
        # splitting only reassociates fp32 sums
        assert np.abs(got - out_f64(base)).max() <= 1e-5, part
    # a partition covering every context is no split at all
    same, ws = prefill_split(c, 2048)
    assert ws is None and torch.equal(same, base)


def test_split_prefill_over_hundreds_of_partitions():
    """Chunks after 4,500 and 4,090 cached tokens at 16-token partitions:
    their last rows span up to 284 partitions, past the 256 whose (max, sum)
    pairs the reduce keeps in lane registers."""
    c = W.prefill_case(97, 8, 2, 128, [(4500, 40), (4090, 8), (0, 20)], dtype="bf16")
    ref = oracle_prefill(c)
    base, _ = prefill_split(c, 0)
    assert np.abs(out_f64(base) - ref).max() <= TOL16
    for part in (16, 32):
        out, ws = prefill_split(c, part)
        assert ws is not None
        assert np.abs(out_f64(out) - ref).max() <= TOL16, part
        assert np.abs(out_f64(out) - out_f64(base)).max() <= 1e-5, part


def test_split_prefill_bf16_output_and_determinism():
    c = W.prefill_case(95, 8, 8, 128, LONG_CHUNKS, dtype="bf16")
    of, _ = prefill_split(c, 256)
    ob, _ = prefill_split(c, 256, out_dtype=torch.bfloat16)
    assert torch.equal(ob.view(torch.int16), of.to(torch.bfloat16).view(torch.int16))
    again, _ = prefill_split(c, 256)
    assert torch.equal(again, of)


def test_split_prefill_rejects_a_small_workspace():
    c = W.prefill_case(96, 4, 4, 64, [(300, 20)], dtype="bf16")
    need = pkv.pkv_prefill_workspace_bytes(20, 4, 64, 320, 64)
    assert need > 0
    small = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(pkv.PkvError):
        prefill_split(c, 64, workspace=small)
    with pytest.raises(pkv.PkvError):
        prefill_split(c, 40)          # not a multiple of 16
