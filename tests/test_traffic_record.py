"""The HBM-traffic records bench.py reports as `roofline.traffic`
(paged_kv_cache_405_amd/traffic.py), on synthetic counter files: per-dispatch
means, the copy calibration's scale, the append kernel left out, a record
replacing the one of the same configuration, and the source digest that makes
a record describe only the code it was measured on."""
import json
import os

from paged_kv_cache_405_amd import traffic as TR


def _csv(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w") as fh:
        fh.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for k, c, v in rows:
            fh.write(f'"{k}",{c},{v}\n')


def _dirs(tmp_path, fetch_kib, write_kib, copy_fetch_kib=524288.0, copy_write_kib=1048576.0):
    dk, ap = "void pa::decode_vec_kernel<pa::f16_t, 128, 16, 1, 4, true>(pa::DecodeParams)", "pa::append_kernel(x)"
    f, w = str(tmp_path / "fetch"), str(tmp_path / "write")
    # two dispatches of the decode kernel (the mean counts), one of the append kernel (left out), one of torch's
    _csv(f, [(dk, "FETCH_SIZE", fetch_kib - 10), (dk, "FETCH_SIZE", fetch_kib + 10), (ap, "FETCH_SIZE", 999.0),
             ("at::native::fill", "FETCH_SIZE", 5.0)])
    _csv(w, [(dk, "WRITE_SIZE", write_kib), (ap, "WRITE_SIZE", 777.0)])
    cf, cw = str(tmp_path / "cf"), str(tmp_path / "cw")
    _csv(cf, [("__amd_rocclr_copyBuffer", "FETCH_SIZE", copy_fetch_kib)])
    _csv(cw, [("__amd_rocclr_copyBuffer", "WRITE_SIZE", copy_write_kib)])
    return f, w, cf, cw, dk


def test_scaling_and_kernel_selection(tmp_path):
    f, w, cf, cw, dk = _dirs(tmp_path, fetch_kib=1000.0, write_kib=64.0)
    path = str(tmp_path / "t.json")
    e = TR.record(path, "llama7b", -1, 1, "bhtd", False, f, w, cf, cw, ["cmd"])
    # the copy moves 1 GiB each way: FETCH_SIZE read as half of it is scaled by 2, WRITE_SIZE by 1
    assert abs(e["fetch_scale"] - 2.0) < 1e-12 and abs(e["write_scale"] - 1.0) < 1e-12
    assert list(e["kernels"]) == [dk]
    assert e["read_bytes_per_call"] == 1000.0 * 1024 * 2
    assert e["write_bytes_per_call"] == 64.0 * 1024
    assert e["bytes_per_call"] == e["read_bytes_per_call"] + e["write_bytes_per_call"]
    assert e["sources_sha256"] == TR.sources_digest()


def test_a_record_replaces_its_configuration_only(tmp_path):
    f, w, cf, cw, _ = _dirs(tmp_path, fetch_kib=1000.0, write_kib=64.0)
    path = str(tmp_path / "t.json")
    TR.record(path, "llama7b", -1, 1, "bhtd", False, f, w, cf, cw, [])
    TR.record(path, "mixed_bs16", -1, 1, "bhtd", False, f, w, cf, cw, [])
    TR.record(path, "shared_prefix", -1, 1, "bhtd", True, f, w, cf, cw, [], prefix_pass=True)
    f2, w2, _, _, _ = _dirs(tmp_path / "again", fetch_kib=2000.0, write_kib=64.0)
    TR.record(path, "llama7b", -1, 1, "bhtd", False, f2, w2, cf, cw, [])
    recs = json.load(open(path))["records"]
    assert sorted(r["workload"] for r in recs) == ["llama7b", "mixed_bs16", "shared_prefix"]
    r7 = TR.lookup("llama7b", -1, 1, "bhtd", path=path)
    assert r7["read_bytes_per_call"] == 2000.0 * 1024 * 2
    # the prefix-pass record answers only for the prefix-pass call
    assert TR.lookup("shared_prefix", -1, 1, "bhtd", True, path=path) is None
    assert TR.lookup("shared_prefix", -1, 1, "bhtd", True, path=path, prefix_pass=True) is not None


def test_a_record_of_other_sources_is_not_reported(tmp_path, monkeypatch):
    f, w, cf, cw, _ = _dirs(tmp_path, fetch_kib=1000.0, write_kib=64.0)
    path = str(tmp_path / "t.json")
    TR.record(path, "llama7b", -1, 1, "bhtd", False, f, w, cf, cw, [])
    assert TR.lookup("llama7b", -1, 1, "bhtd", path=path) is not None
    monkeypatch.setattr(TR, "sources_digest", lambda: "0" * 64)
    assert TR.lookup("llama7b", -1, 1, "bhtd", path=path) is None
    assert TR.lookup("llama7b", -1, 1, "bhtd", path=str(tmp_path / "missing.json")) is None


def test_the_digest_covers_every_kernel_source():
    files = sorted(os.listdir(os.path.join(TR.PKG, "csrc")))
    assert any(n.endswith(".hip") for n in files) and any(n.endswith(".h") for n in files)
    d1 = TR.sources_digest()
    assert d1 == TR.sources_digest() and len(d1) == 64
