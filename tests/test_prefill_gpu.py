"""GPU parity of multi-token paged attention (pa_prefill) against the fp64
oracle (oracle/prefill.py): from-scratch prefills, chunks over a cached
history, single rows (decode), chunks longer than their context, every block
size, both head dims and group shapes from MHA to 32 q heads per kv head;
the append-then-attend flow of a chunked prefill; and the rows that
query_start leaves outside q are never touched."""
import numpy as np
import pytest
import torch

import oracle
from oracle.prefill import paged_prefill
from paged_kv_cache_405_amd import binding as B
from paged_kv_cache_405_amd import workloads as W
from tests.pa_harness import assert_close, compare, log, to_dev, upload

pytestmark = pytest.mark.gpu


def _starts(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def _run(w, g, q_np, counts, shared=False):
    qs = _starts(counts)
    q = to_dev(q_np, w.dtype)
    out = torch.full_like(q, float("nan"))
    B.pa_prefill(out, q, g.k_cache, g.v_cache, g.tables, g.ctx, torch.from_numpy(qs).cuda(), max(counts), w.scale,
                 layout=g.layout, num_blocks=w.num_blocks, shared_blocks=shared)
    torch.cuda.synchronize()
    ref = paged_prefill(q_np, w.k_cache, w.v_cache, w.block_tables, w.context_lens, qs, w.scale, w.dtype)
    return out, ref


def _shapes():
    out = []
    for dtype in ("f16", "bf16"):
        for D in (128, 256):
            for bs in (8, 16, 32):
                for Hq, Hkv in ((8, 8), (16, 4), (64, 8), (16, 1), (32, 1)):
                    if D == 256 and (Hq, Hkv) in ((64, 8), (32, 1)):
                        continue        # keep the oracle quick
                    out.append((dtype, D, bs, Hq, Hkv))
    return out


@pytest.mark.parametrize("dtype,D,bs,Hq,Hkv", _shapes())
def test_prefill_matches_the_oracle(dtype, D, bs, Hq, Hkv):
    # contexts and their query rows: from scratch, chunks over a history, a single row, a ragged tail
    ctxs = [37, 100, 1, 64, 130, 17]
    counts = [37, 20, 1, 5, 33, 17]
    w = W.custom(f"prefill_{dtype}_{D}_{bs}_{Hq}x{Hkv}", dtype, ctxs, Hq, Hkv, D, bs,
                 seed=D + 3 * bs + Hq + Hkv, append=False, table_pad=1)
    rng = np.random.default_rng(D * bs + Hq)
    q_np = W.to_storage(rng.standard_normal((sum(counts), Hq, D), dtype=np.float32), dtype)
    g = upload(w)
    log(f"[gpu] prefill {w.name}")
    out, ref = _run(w, g, q_np, counts)
    assert_close(compare(out, ref, dtype), dtype, w.name)


def test_rows_past_the_context_are_zero_and_bad_starts_touch_nothing():
    w = W.custom("prefill_edges", "bf16", [3, 0, 40], 16, 4, 128, 16, seed=77, append=False)
    rng = np.random.default_rng(78)
    counts = [6, 2, 9]
    q_np = W.to_storage(rng.standard_normal((sum(counts), 16, 128), dtype=np.float32), "bf16")
    g = upload(w)
    out, ref = _run(w, g, q_np, counts)
    assert_close(compare(out, ref, "bf16"), "bf16", "prefill edges")
    assert not out[:3].any() and not out[6:8].any()       # positions before 0, an empty context
    # query_start pointing outside q: those rows are skipped, the others still computed
    qs = torch.tensor([0, 6, 8, 40], dtype=torch.int32, device="cuda")      # the last sequence runs past total_q
    q = to_dev(q_np, "bf16")
    out2 = torch.full_like(q, 7.0)
    B.pa_prefill(out2, q, g.k_cache, g.v_cache, g.tables, g.ctx, qs, 32, w.scale, num_blocks=w.num_blocks)
    torch.cuda.synchronize()
    # the sequence that claims rows past q keeps the 9 rows inside it, as if it had asked for 9
    assert torch.equal(out2, out)


def test_one_row_is_decode_and_the_cache_policy_changes_no_bit():
    w = W.custom("prefill_decode", "f16", [1, 50, 300, 17], 32, 8, 128, 16, seed=91, append=False)
    g = upload(w)
    counts = [1, 1, 1, 1]
    out, ref = _run(w, g, w.q, counts)
    assert_close(compare(out, ref, "f16"), "f16", "prefill of one row")
    dec = torch.empty_like(out)
    B.pa_decode_ex(dec, to_dev(w.q, "f16"), g.k_cache, g.v_cache, g.tables, g.ctx, w.scale,
                   num_blocks=w.num_blocks, kernel=B.PA_KERNEL_MFMA, partition_tokens=B.PA_PARTITION_SINGLE)
    torch.cuda.synchronize()
    assert_close(compare(dec, oracle.paged_decode(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens,
                                                  w.scale, "f16"), "f16"), "f16", "decode of the same rows")
    shared, _ = _run(w, g, w.q, counts, shared=True)
    assert torch.equal(shared, out)


@pytest.mark.parametrize("dtype,Hq,Hkv", [("f16", 32, 32), ("bf16", 64, 8)])
def test_chunked_prefill_append_then_attend(dtype, Hq, Hkv):
    # a 3-chunk prompt: each chunk's K/V appended at its slots, then the chunk attends its history
    D, bs, NB = 128, 16, 40
    rng = np.random.default_rng(Hq)
    prompt = [50, 30, 45]
    total = sum(prompt)
    k_all = W.to_storage(rng.standard_normal((total, Hkv, D), dtype=np.float32), dtype)
    v_all = W.to_storage(rng.standard_normal((total, Hkv, D), dtype=np.float32), dtype)
    q_all = W.to_storage(rng.standard_normal((total, Hq, D), dtype=np.float32), dtype)
    phys = rng.permutation(NB)[:-(-total // bs)].astype(np.int32)
    table = np.full((1, 16), -1, np.int32)
    table[0, :len(phys)] = phys
    kc = W.to_storage(np.full((NB, bs, Hkv, D), np.nan, dtype=np.float32), dtype)   # unwritten slots are NaN
    vc = kc.copy()
    g_k = B.to_layout(to_dev(kc, dtype), B.PA_LAYOUT_BHTD)
    g_v = B.to_layout(to_dev(vc, dtype), B.PA_LAYOUT_BHTD)
    scale = float(np.float32(1 / np.sqrt(D)))
    done = 0
    for n in prompt:
        pos = np.arange(done, done + n)
        slots = (phys[pos // bs].astype(np.int64) * bs + pos % bs)
        B.pa_reshape_and_cache(to_dev(k_all[pos], dtype), to_dev(v_all[pos], dtype), g_k, g_v,
                               torch.from_numpy(slots).cuda())
        oracle.reshape_and_cache(k_all[pos], v_all[pos], kc, vc, slots, dtype)
        done += n
        ctx = np.array([done], np.int32)
        q = to_dev(q_all[pos], dtype)
        out = torch.empty_like(q)
        B.pa_prefill(out, q, g_k, g_v, torch.from_numpy(table).cuda(), torch.from_numpy(ctx).cuda(),
                     torch.tensor([0, n], dtype=torch.int32, device="cuda"), n, scale, num_blocks=NB)
        torch.cuda.synchronize()
        ref = paged_prefill(q_all[pos], kc, vc, table, ctx, np.array([0, n], np.int32), scale, dtype)
        assert_close(compare(out, ref, dtype), dtype, f"chunk ending at {done}")
