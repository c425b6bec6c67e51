"""GPU parity of each decode kernel, forced through pa_decode_ex's `kernel`
argument, against the fp64 CPU oracle on the same seeded inputs.

The vector kernel covers every shape; the matrix-core (MFMA) kernel covers
f16/bf16 with head_dim 128 or 256 and any q-head group that fills at most 16
columns per workgroup (or a multiple of 16).  Both must meet the same bounds
as the default path (fp16/bf16: max-abs <= 2e-3, relative L2 <= 1e-3 against
the oracle rounded to the output type).  Lengths are ragged around tile
(16 tokens), block and partition edges; partitions include ones that are not
a multiple of the 16-token tile (block size 8), so a tile can straddle two
partitions.
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_405_amd import binding as B
from paged_kv_cache_405_amd import workloads as W
from tests.pa_harness import assert_close, compare, gpu_step, log, oracle_step, upload

pytestmark = pytest.mark.gpu

GROUPS = [(4, 4), (6, 2), (8, 1), (16, 2), (32, 2), (64, 2)]


def _mfma_cases():
    cases = []
    for dtype in ("f16", "bf16"):
        for D in (128, 256):
            for bs in (8, 16, 32):
                for Hq, Hkv in GROUPS:
                    cases.append((dtype, D, bs, Hq, Hkv))
    return cases


@pytest.mark.parametrize("dtype,D,bs,Hq,Hkv", _mfma_cases())
def test_mfma_kernel_ragged(dtype, D, bs, Hq, Hkv):
    ctxs = [1, 5, 15, 16, 17, bs + 3, 2 * bs, 47, 100, 256, 257, 600]
    w = W.custom(f"mfma_{dtype}_{D}_{bs}_{Hq}x{Hkv}", dtype, ctxs, Hq, Hkv, D, bs,
                 seed=1000 + D + bs * 3 + Hq, append=True, table_pad=2)
    log(f"[gpu] {w.name}")
    g = upload(w)
    ref = oracle_step(w)
    first = True
    for pt in (-1, 0, -2, bs, 4 * bs, 256):
        out = gpu_step(w, g, partition_tokens=pt, append=first, kernel=B.PA_KERNEL_MFMA)
        first = False
        torch.cuda.synchronize()
        assert_close(compare(out, ref, dtype), dtype, f"{w.name} mfma pt={pt}")


@pytest.mark.parametrize("kernel", [B.PA_KERNEL_VECTOR, B.PA_KERNEL_MFMA])
@pytest.mark.parametrize("name", ["llama70b_gqa", "llama7b"])
def test_forced_kernel_full_workload(name, kernel):
    """Both kernels on the full grouped-query (70B-shaped) and MHA (7B-shaped)
    workloads, in the configuration the benchmark times."""
    w = W.WORKLOADS[name]()
    log(f"[gpu] {name} kernel {kernel}")
    g = upload(w)
    out = gpu_step(w, g, partition_tokens=w.partition_tokens, kernel=kernel)
    torch.cuda.synchronize()
    assert_close(compare(out, oracle_step(w), w.dtype), w.dtype, f"{name} kernel={kernel}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_mfma_context_zero_and_one(dtype):
    """ctx = 0 gives a zero row; ctx = 1 gives V[0] bit for bit (p = 1, l = 1)."""
    w = W.custom(f"mfma_edge_{dtype}", dtype, [0, 1, 0, 1, 33], 16, 2, 128, 16, seed=15, append=False)
    g = upload(w)
    for pt in (-1, 0, -2, 16):
        out = gpu_step(w, g, partition_tokens=pt, append=False, kernel=B.PA_KERNEL_MFMA)
        torch.cuda.synchronize()
        got = out.cpu()
        assert torch.all(got[0] == 0) and torch.all(got[2] == 0)
        for s in (1, 3):
            b = int(w.block_tables[s, 0])
            for h in range(16):
                row = np.ascontiguousarray(w.v_cache[b, 0, h // 8])
                want = torch.from_numpy(row.view(np.int16)).view(torch.bfloat16) if dtype == "bf16" \
                    else torch.from_numpy(row)
                assert torch.equal(got[s, h], want), f"seq {s} head {h}"


def test_mfma_unmapped_block_and_rerun():
    """An unmapped table entry contributes nothing; reruns are bit-identical."""
    w = W.custom("mfma_unmapped", "bf16", [40, 70, 300], 8, 1, 128, 16, seed=21, append=False)
    tables = w.block_tables.copy()
    last = (70 + 15) // 16 - 1
    tables[1, last] = -5
    g = upload(w)
    import dataclasses
    g2 = dataclasses.replace(g, tables=torch.from_numpy(tables).cuda())
    a = gpu_step(w, g2, partition_tokens=-1, append=False, kernel=B.PA_KERNEL_MFMA, num_blocks=w.num_blocks)
    b = gpu_step(w, g2, partition_tokens=-1, append=False, kernel=B.PA_KERNEL_MFMA, num_blocks=w.num_blocks)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = oracle_step(w, append=False, context_lens=np.array([40, last * 16, 300], dtype=np.int32))
    assert_close(compare(a, ref, "bf16"), "bf16", "mfma unmapped last block")
