"""GPU parity of the entry points and shapes the benchmark times.

- The bare `pa_decode` (the interface's plain signature: cache layout
  [NB, Hkv, bs, D], the library's own partition and kernel, a workspace the
  binding sizes and allocates) on the tiny workload and at full size on the
  Llama-2-7B- and Llama-2-70B-shaped workloads, element by element against
  the fp64 oracle, and bit for bit against pa_decode_ex on the same path.
- `pa_prefill` at the shape `bench.py --op prefill` times: 16 sequences, each
  a 512-row chunk over 1536 cached tokens (context 2048), 32 x 128 MHA, fp16,
  block size 16.  The GPU computes the whole batch; the oracle checks every
  row of a sample of sequences (first, middle, last), each sequence's blocks
  copied into a small pool so the oracle decodes only what it reads.
- `pa_prefill`, and `pa_prefill_shared_prefix` (the call the benchmark
  times), at the shape of the prefix-cache call `bench.py --op prefix_cache`:
  127 requests whose tables start with the same 94 blocks (a 1504-token
  system prompt) and whose 8-200 own tokens are the query rows.

Pages: "vLLM 与 PagedAttention" section 二 ("注意力计算改造": the decode
call), section 四 (prefix caching) and section 六 ("关键的工程优化":
chunked prefill).
"""
import numpy as np
import pytest
import torch

from oracle.prefill import paged_prefill
from paged_kv_cache_405_amd import binding as B
from paged_kv_cache_405_amd import workloads as W
from tests.pa_harness import assert_close, compare, log, oracle_step, to_dev, upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny_f32", "llama7b", "llama70b_gqa"])
def test_bare_pa_decode(name):
    """append, then the bare pa_decode with workspace=None (the binding asks the
    library for the size and allocates it)"""
    w = W.WORKLOADS[name]()
    log(f"[gpu] bare pa_decode {name}: {w.description}")
    g = upload(w, B.PA_LAYOUT_BHTD)
    B.pa_reshape_and_cache(g.new_k, g.new_v, g.k_cache, g.v_cache, g.slots)
    out = torch.full_like(g.q, float("nan"))
    B.pa_decode(out, g.q, g.k_cache, g.v_cache, g.tables, g.ctx, w.scale)
    ex = torch.full_like(g.q, float("nan"))
    B.pa_decode_ex(ex, g.q, g.k_cache, g.v_cache, g.tables, g.ctx, w.scale)
    torch.cuda.synchronize()
    assert_close(compare(out, oracle_step(w), w.dtype), w.dtype, f"bare pa_decode {name}")
    assert torch.equal(out, ex), "pa_decode and pa_decode_ex (automatic path) differ"


def _compact(w, seqs):
    """The listed sequences' blocks copied into a pool of their own, with
    tables renumbered to it (numpy only: what the oracle then reads)."""
    bs = w.block_size
    tabs = []
    blocks = []
    for s in seqs:
        n = W.blocks_needed(int(w.context_lens[s]), bs)
        tabs.append(list(range(len(blocks), len(blocks) + n)))
        blocks.extend(int(b) for b in w.block_tables[s, :n])
    MB = max(len(t) for t in tabs)
    table = np.full((len(seqs), MB), -1, np.int32)
    for i, t in enumerate(tabs):
        table[i, :len(t)] = t
    idx = np.array(blocks, dtype=np.int64)
    return w.k_cache[idx], w.v_cache[idx], table, w.context_lens[list(seqs)]


def _check_sample(w, q_np, counts, out, seqs, what):
    starts = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    kc, vc, table, ctx = _compact(w, seqs)
    rows = np.concatenate([np.arange(starts[s], starts[s + 1]) for s in seqs])
    sub_counts = [int(counts[s]) for s in seqs]
    qs = np.concatenate([[0], np.cumsum(sub_counts)]).astype(np.int32)
    ref = paged_prefill(q_np[rows], kc, vc, table, ctx, qs, w.scale, w.dtype)
    got = out[torch.from_numpy(rows).cuda()]
    assert_close(compare(got, ref, w.dtype), w.dtype, what)


def test_prefill_at_the_benchmarked_shape():
    S, chunk, hist, H, D, bs = 16, 512, 1536, 32, 128, 16
    w = W.custom("prefill_bench_shape", "f16", [hist + chunk] * S, H, H, D, bs, seed=21, append=False)
    rng = np.random.default_rng(22)
    q_np = W.to_storage(rng.standard_normal((S * chunk, H, D), dtype=np.float32), "f16")
    counts = np.full(S, chunk)
    g = upload(w)
    q = to_dev(q_np, "f16")
    out = torch.full_like(q, float("nan"))
    qs = torch.arange(0, S * chunk + 1, chunk, dtype=torch.int32, device="cuda")
    log(f"[gpu] prefill at the benchmarked shape: {S} x {chunk} rows over {hist} cached tokens, {H}x{D} f16")
    B.pa_prefill(out, q, g.k_cache, g.v_cache, g.tables, g.ctx, qs, chunk, w.scale, num_blocks=w.num_blocks)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all(), "rows left unwritten or non-finite"
    _check_sample(w, q_np, counts, out, [0, S // 2, S - 1], "prefill 16 x 512 over 1536")


def _prefix_cache_call(shared):
    """127 requests after the first: each attends the 94 shared blocks plus its
    own 8-200 tokens, whose rows are the query rows (the cache supplied the rest)."""
    S, H, D, bs, prefix_blocks = 127, 32, 128, 16, 94
    rng = np.random.default_rng(31)
    own = rng.integers(8, 201, S)
    ctxs = prefix_blocks * bs + own
    w = W.custom("prefix_cache_call_shape", "f16", ctxs, H, H, D, bs, seed=33, append=False,
                 shared_prefix_blocks=prefix_blocks)
    assert (w.block_tables[:, :prefix_blocks] == w.block_tables[0, :prefix_blocks]).all()
    q_np = W.to_storage(rng.standard_normal((int(own.sum()), H, D), dtype=np.float32), "f16")
    g = upload(w)
    q = to_dev(q_np, "f16")
    out = torch.full_like(q, float("nan"))
    qs = torch.from_numpy(np.concatenate([[0], np.cumsum(own)]).astype(np.int32)).cuda()
    log(f"[gpu] prefill at the prefix-cache call shape ({'shared prefix' if shared else 'per request'}): "
        f"{S} requests, {int(own.sum())} rows")
    if shared:
        B.pa_prefill_shared_prefix(out, q, g.k_cache, g.v_cache, g.tables, g.ctx, qs, int(own.max()), w.scale,
                                   prefix_blocks, num_blocks=w.num_blocks)
    else:
        B.pa_prefill(out, q, g.k_cache, g.v_cache, g.tables, g.ctx, qs, int(own.max()), w.scale,
                     num_blocks=w.num_blocks)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all(), "rows left unwritten or non-finite"
    short, long_ = int(np.argmin(own)), int(np.argmax(own))
    _check_sample(w, q_np, own, out, sorted({0, short, long_, S // 2, S - 1}),
                  "prefix-cache call shape" + (", shared prefix" if shared else ""))


def test_prefill_at_the_prefix_cache_call_shape():
    _prefix_cache_call(False)


def test_shared_prefix_prefill_at_the_prefix_cache_call_shape():
    """pa_prefill_shared_prefix, the call the prefix-cache benchmark times, on the same inputs."""
    _prefix_cache_call(True)
