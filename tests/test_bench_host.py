"""Host logic of bench.py (no GPU): the algorithmic bytes and flops behind its roofline
object, and the lookup of the committed FC1 traffic counters (profiles/fc1_<workload>_pmc.md),
which must be withdrawn as soon as a kernel source they were taken on changes."""
import os
import shutil

import bench
import lmoe_inputs as LI

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_fc1_bytes_decode_and_mx_shapes():
    dec = LI.CONFIGS["decode_bf16"]
    # 114 touched experts: W1 (2d x L, bf16) once each, the 8 latent rows, 114 tiles of 16
    # activation rows written
    assert bench.fc1_bytes(dec, 114, 114 * 16) == 114 * 1024 * 2048 * 2 + 8 * 2048 * 2 + 1824 * 512 * 2
    assert bench.fc1_bytes(dec, 114, 114 * 16) == 480051200
    mx = LI.CONFIGS["mx_experts"]
    # MXFP4: half a byte per weight + one e8m0 byte per 32; MXFP8 rows: one byte per element
    # + one per 32 (764 touched experts, 990 tiles of 32 rows)
    want = 764 * 1024 * 2048 * 17 // 32 + 1024 * 2048 * 33 // 32 + 31680 * 512 * 33 // 32
    assert bench.fc1_bytes(mx, 764, 31680) == want == 870071296


def test_fc1_roofline_bound_by_workload():
    pf = LI.CONFIGS["prefill_bf16"]
    r = bench.fc1_roofline(pf, 692, 188288, 131072, 1.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["algorithmic_flops"] == 2 * 131072 * 1024 * 2048      # pairs, not padded rows
    assert abs(r["achieved"] - 2 * 131072 * 1024 * 2048 / 1e-3 / 1e12) < 0.1
    dec = LI.CONFIGS["decode_bf16"]
    r = bench.fc1_roofline(dec, 114, 1824, 128, 0.08)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["achieved"] - 480051200 / 0.08e-3 / 1e9) < 0.1
    assert abs(r["frac"] - r["achieved"] / 8000.0) < 1e-4
    # the kernel named is the one each workload's FC1 launches (the profiles name the same)
    assert "tiled_gemm_kernel" in bench.fc1_roofline(pf, 692, 188288, 131072, 1.0)["kernel"]
    assert "stream_gemm_kernel" in r["kernel"]
    mx = LI.CONFIGS["mx_experts"]
    assert mx.tile_m == 32 and "mx_fc1_lds_kernel" in bench.fc1_roofline(mx, 764, 31680, 16384, 0.2)["kernel"]


def _profile_copy(tmp_path, name):
    """A copy of the committed counter profile of `name` (with its kernel sources) under
    tmp_path, its recorded hash set to the sources as they are now; returns the recorded
    traffic line."""
    import hashlib
    prof = os.path.join("profiles", f"fc1_{name}_pmc.md")
    with open(os.path.join(ROOT, prof)) as f:
        text = f.read()
    srcs = next(l for l in text.splitlines() if l.startswith("kernel_sources:")).split(":", 1)[1].split()
    h = hashlib.sha256()
    for rel in srcs:
        os.makedirs(tmp_path / os.path.dirname(rel), exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), tmp_path / rel)
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    lines = [l if not l.startswith("kernel_sources_sha256:") else f"kernel_sources_sha256: {h.hexdigest()}"
             for l in text.splitlines()]
    os.makedirs(tmp_path / "profiles", exist_ok=True)
    with open(tmp_path / prof, "w") as f:
        f.write("\n".join(lines) + "\n")
    return next(l for l in lines if l.startswith("traffic_bytes_per_launch:"))


def test_fc1_traffic_reads_each_committed_profile(tmp_path, monkeypatch):
    """The lookup parses every committed profile (here with its hash matched to the
    current sources; the real files are withdrawn by the next test's rule whenever a
    kernel source has changed since they were taken)."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    for name in ("decode_bf16", "prefill_bf16", "mx_experts"):
        line = _profile_copy(tmp_path, name)
        cfg = LI.CONFIGS[name]
        v = bench.fc1_traffic(cfg, 2)
        assert isinstance(v, int) and v > 0, name
        assert line == f"traffic_bytes_per_launch: {v}"
        assert bench.fc1_traffic(cfg, 3) is None      # counters were taken at seed 2 only


def test_fc1_traffic_is_withdrawn_when_a_kernel_source_changes(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _profile_copy(tmp_path, "decode_bf16")
    cfg = LI.CONFIGS["decode_bf16"]
    assert bench.fc1_traffic(cfg, 2) is not None
    with open(os.path.join(ROOT, "profiles", "fc1_decode_bf16_pmc.md")) as f:
        srcs = next(l for l in f if l.startswith("kernel_sources:")).split(":", 1)[1].split()
    with open(tmp_path / srcs[0], "a") as f:
        f.write("\n// edited\n")
    assert bench.fc1_traffic(cfg, 2) is None


def test_expert_floor_and_layer_flops():
    pf = LI.CONFIGS["prefill_bf16"]
    # a heavy expert (4000 rows) is MFMA-bound, a light one (3 rows) HBM-bound; the floor
    # takes the larger of the two times per expert and sums over the experts
    c = 4000
    flops = 2.0 * c * 1024 * 2048
    nbytes = 1024 * 2048 * 2 + c * 2048 * 2 + c * 512 * 2
    want = max(flops / 2.5e15, nbytes / 8e12) * 1e3
    assert abs(bench.fc1_expert_floor_ms(pf, [c]) - want) < 1e-12
    light = 3
    want_light = max(2.0 * light * 1024 * 2048 / 2.5e15, (1024 * 2048 * 2 + light * 2560 * 2) / 8e12) * 1e3
    assert abs(bench.fc1_expert_floor_ms(pf, [c, 0, light]) - (want + want_light)) < 1e-12
    r = bench.fc1_roofline(pf, 2, 4224, c + light, 1.0, [c, 0, light])
    assert abs(r["expert_floor_frac"] - (want + want_light)) < 1e-4
    # dense projections over all tokens plus the routed FC1 + FC2 over the pairs
    dense = 2 * 8192 * (896 * 7168 + 2048 * 7168 + 3 * 7168 * 4096 + 7168 * 2048)
    assert bench.layer_flops(pf) == dense + 2 * 8192 * 16 * 3 * 2048 * 512


def test_percentiles_nearest_rank():
    p = bench.percentiles([5.0, 1.0, 4.0, 2.0, 3.0] * 2 + [100.0])
    assert p["median"] == 3.0 and p["p10"] == 1.0 and p["p90"] == 5.0


def test_bench_refuses_several_gpus():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2 and "one GPU" in r.stderr
