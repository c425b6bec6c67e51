"""bench.py's host-side settings for every workload it offers (no device):
the arguments parse, the workloads carry what the run reads, and the cache
hint follows the workload's sharing."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from paged_kv_cache_405_amd import binding as B  # noqa: E402
from paged_kv_cache_405_amd import workloads as W  # noqa: E402

BENCH_WORKLOADS = ["llama7b", "llama70b_gqa", "llama70b_tp8", "mixed_bs8", "mixed_bs16", "mixed_bs32",
                   "shared_prefix"]


@pytest.fixture(scope="module")
def made():
    # the smallest instances of each shape keep this quick
    small = {"llama7b": dict(num_seqs=2), "llama70b_gqa": dict(num_seqs=2), "llama70b_tp8": dict(num_seqs=2),
             "shared_prefix": dict(num_seqs=2),
             "mixed_bs8": dict(num_seqs=4), "mixed_bs16": dict(num_seqs=4), "mixed_bs32": dict(num_seqs=4)}
    out = {}
    for name in BENCH_WORKLOADS:
        kw = dict(poison=False)
        kw.update(small.get(name, {}))
        out[name] = W.WORKLOADS[name](**kw)
    return out


@pytest.mark.parametrize("name", BENCH_WORKLOADS)
def test_default_run_settings(made, name):
    args = bench.parse(["--workload", name])
    w = made[name]
    cfg = bench.run_config(args, w, B)
    assert cfg["pt"] == B.PA_PARTITION_AUTO and cfg["kern"] == B.PA_KERNEL_AUTO
    assert cfg["layers"] == (80 if name.startswith("llama70b") else 32)
    assert cfg["shared"] == (name == "shared_prefix")
    # what the timed loop reads from the workload
    for attr in ("block_tables", "context_lens", "slot_mapping", "new_k", "new_v", "q", "scale",
                 "max_blocks_per_seq", "num_kv_heads", "block_size"):
        assert getattr(w, attr) is not None
    assert w.kv_bytes() > 0


def test_flags_and_overrides(made):
    w = made["shared_prefix"]
    assert not bench.run_config(bench.parse(["--shared-blocks", "off"]), w, B)["shared"]
    assert bench.run_config(bench.parse(["--shared-blocks", "on"]), made["llama7b"], B)["shared"]
    cfg = bench.run_config(bench.parse(["--partition-tokens", "512", "--kernel", "mfma", "--layout", "bthd",
                                        "--layers", "3"]), made["llama70b_gqa"], B)
    assert (cfg["pt"], cfg["kern"], cfg["layout"], cfg["layers"]) == (512, B.PA_KERNEL_MFMA, B.PA_LAYOUT_BTHD, 3)


def test_default_workload_is_the_7b_shape():
    assert bench.parse([]).workload == "llama7b"


def test_warmup_defaults():
    """the matrix-core bound ops warm up longer by default; an explicit --warmup always wins"""
    assert bench.parse([]).warmup == 3
    assert bench.parse(["--op", "copy_blocks"]).warmup == 3
    assert bench.parse(["--op", "prefill"]).warmup == 20
    assert bench.parse(["--op", "prefix_cache"]).warmup == 20
    assert bench.parse(["--op", "prefill", "--warmup", "2"]).warmup == 2
    assert bench.parse(["--config-warmup", "4"]).config_warmup == 4


def test_cpu_rates_on_a_small_workload():
    """the oracle timing helper: median of its samples, positive rates, the thread count it used"""
    w = W.tiny_f32(poison=False)
    r = bench.cpu_rates(w, 0.05, runs=3)
    assert r["runs"] == 3 and len(r["values"]) == 3 and r["value"] == sorted(r["values"])[1]
    assert r["value"] > 0 and r["seq_layers_per_s"] > 0 and r["threads"] >= 1
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()


def test_config_list_covers_the_five_workloads():
    assert {"tiny_f32", "llama7b", "mixed_bs8", "mixed_bs16", "mixed_bs32", "shared_prefix",
            "llama70b_gqa"} <= set(bench.CONFIG_WORKLOADS)
    a = bench.parse(["--no-configs", "--no-probe", "--config-steps", "2"])
    assert a.no_configs and a.no_probe and a.config_steps == 2
