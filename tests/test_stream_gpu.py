"""GPU parity of the balanced schedule (partition_tokens = 0, the library's
default): every wave of the GPU takes an equal share of the token stream, a
unit cut between waves leaves pieces, and a reduce kernel merges them.

Cases aimed at the schedule itself: one long sequence cut across hundreds of
waves (long piece chains), fewer steps than waves (idle waves), empty contexts
in between (zero rows written by exactly one wave), reproducible bits, and
the exact workspace size."""
import ctypes

import numpy as np
import pytest
import torch

from paged_kv_cache_405_amd import binding as B
from paged_kv_cache_405_amd import workloads as W
from tests.pa_harness import assert_close, compare, gpu_step, log, oracle_step, upload

pytestmark = pytest.mark.gpu

KERNELS = [B.PA_KERNEL_VECTOR, B.PA_KERNEL_MFMA]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_one_long_sequence_cut_across_many_waves(dtype, kernel):
    w = W.custom(f"stream_long_{dtype}", dtype, [8191], 16, 2, 128, 16, seed=31, append=True)
    log(f"[gpu] {w.name} kernel {kernel}")
    g = upload(w)
    out = gpu_step(w, g, partition_tokens=B.PA_PARTITION_BALANCED, kernel=kernel)
    torch.cuda.synchronize()
    assert_close(compare(out, oracle_step(w), dtype), dtype, f"{w.name} kernel={kernel}")


@pytest.mark.parametrize("kernel", KERNELS)
def test_empty_contexts_and_idle_waves(kernel):
    ctxs = [0, 3, 0, 0, 17, 1, 0, 40, 0]
    w = W.custom("stream_sparse", "bf16", ctxs, 8, 1, 128, 16, seed=32, append=False)
    log(f"[gpu] {w.name} kernel {kernel}")
    g = upload(w)
    out = gpu_step(w, g, partition_tokens=B.PA_PARTITION_BALANCED, append=False, kernel=kernel)
    torch.cuda.synchronize()
    got = out.cpu()
    for s, c in enumerate(ctxs):
        if c == 0:
            assert torch.all(got[s] == 0), f"seq {s}"
    assert_close(compare(out, oracle_step(w, append=False), "bf16"), "bf16", f"{w.name} kernel={kernel}")


@pytest.mark.parametrize("dtype,D,bs,Hq,Hkv", [("f32", 32, 16, 2, 2), ("f32", 64, 8, 4, 2), ("f16", 256, 32, 4, 4),
                                               ("bf16", 64, 16, 8, 8), ("f16", 128, 8, 32, 32)])
def test_vector_shapes_balanced(dtype, D, bs, Hq, Hkv):
    ctxs = [1, 2 * bs - 1, 300, 0, 1000, 47, 129, 5]
    w = W.custom(f"stream_vec_{dtype}_{D}_{bs}_{Hq}x{Hkv}", dtype, ctxs, Hq, Hkv, D, bs,
                 seed=40 + D + bs, append=False, table_pad=1)
    log(f"[gpu] {w.name}")
    g = upload(w)
    out = gpu_step(w, g, partition_tokens=B.PA_PARTITION_BALANCED, append=False, kernel=B.PA_KERNEL_VECTOR)
    torch.cuda.synchronize()
    assert_close(compare(out, oracle_step(w, append=False), dtype), dtype, w.name)


@pytest.mark.parametrize("name", ["llama7b", "llama70b_gqa", "shared_prefix"])
def test_balanced_rerun_bit_identical(name):
    w = W.WORKLOADS[name]()
    log(f"[gpu] {name} balanced reruns")
    g = upload(w)
    a = gpu_step(w, g, partition_tokens=B.PA_PARTITION_BALANCED)
    b = gpu_step(w, g, partition_tokens=B.PA_PARTITION_BALANCED, append=False)
    c = gpu_step(w, g, partition_tokens=B.PA_PARTITION_BALANCED, append=False)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)
    assert_close(compare(a, oracle_step(w), w.dtype), w.dtype, f"{name} balanced")


def test_workspace_exact_size():
    w = W.custom("stream_ws", "f16", [100, 2000, 7], 32, 8, 128, 16, seed=33, append=False)
    g = upload(w)
    S, Hq, D = w.q.shape
    bal = B.PA_PARTITION_BALANCED
    need = B.pa_decode_workspace_bytes(S, Hq, w.num_kv_heads, D, w.block_size, w.max_blocks_per_seq, B.PA_F16, bal)
    # (max, sum) pairs and partial outputs of the two piece slots of at least 8 waves
    assert need >= 2 * 8 * (4 + 8 + D * 4)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(g.q)
    L = B.lib()
    args = lambda nbytes, kern: (out.data_ptr(), g.q.data_ptr(), g.k_cache.data_ptr(), g.v_cache.data_ptr(),  # noqa
                                 g.tables.data_ptr(), g.ctx.data_ptr(), S, Hq, w.num_kv_heads, D, w.block_size,
                                 w.max_blocks_per_seq, w.num_blocks, ctypes.c_float(w.scale), B.PA_F16,
                                 B.PA_LAYOUT_BHTD, bal, kern, 0, ws.data_ptr(), nbytes, ctypes.c_void_p(
                                     torch.cuda.current_stream().cuda_stream))
    # the query covers whichever kernel the call takes: enough for both, exactly enough for the larger
    kernels = (B.PA_KERNEL_AUTO, B.PA_KERNEL_VECTOR, B.PA_KERNEL_MFMA)
    short = [L.pa_decode_ex(*args(need - 1, k)) for k in kernels]
    torch.cuda.synchronize()
    assert B.PA_ERR_WORKSPACE in short and set(short) <= {B.PA_OK, B.PA_ERR_WORKSPACE}
    ref = oracle_step(w, append=False)
    for k in kernels:
        out.fill_(float("nan"))
        assert L.pa_decode_ex(*args(need, k)) == B.PA_OK
        torch.cuda.synchronize()
        assert_close(compare(out, ref, "f16"), "f16", f"exact workspace, kernel {k}")
