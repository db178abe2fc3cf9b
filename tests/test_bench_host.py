"""Host logic of bench.py that runs without a GPU: the one-GPU guard and the
lookup of committed HBM counter figures, which must be dropped once a
kernel's sources or the layer shape differ from the ones they were taken on."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_comment_edits_do_not_change_the_source_hash():
    code = "int f(int x) {\n  return x + 1;\n}\n"
    noted = "// adds one\nint f(int x) {  /* the\n argument */\n  return x + 1;   // plus one\n}\n\n"
    assert bench._code_only(code) == bench._code_only(noted)
    assert bench._code_only(code) != bench._code_only(code.replace("+ 1", "+ 2"))


def _write_traffic(tmp_path, kernel, source_hash, shape, nbytes):
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps({"kernels": {kernel: {"source_hash": source_hash, "shape": shape,
                                                     "bytes_per_launch": nbytes}}}))
    return str(path)


def test_traffic_is_used_only_on_matching_sources_and_shape(tmp_path, monkeypatch):
    kernel, shape = "dD_gemm", [4096, 11008, 2048]
    current = bench.kernel_source_hash(kernel)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _write_traffic(tmp_path, kernel, current, shape, 12345))
    assert bench.measured_traffic(kernel, shape) == 12345
    assert bench.measured_traffic(kernel, [4096, 4096, 2048]) is None          # another layer
    assert bench.measured_traffic("error_gemm", shape) is None                  # no entry
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _write_traffic(tmp_path, kernel, "0" * 16, shape, 12345))
    assert bench.measured_traffic(kernel, shape) is None                        # stale sources
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic(kernel, shape) is None


def test_every_profiled_role_names_existing_sources():
    for kernel, files in bench.KERNEL_SOURCES.items():
        for f in files:
            assert os.path.exists(os.path.join(ROOT, "learnable_channel_permutation_amd", "csrc", f)), (kernel, f)
        assert len(bench.kernel_source_hash(kernel)) == 16


def test_kernel_work_of_the_bench_layer():
    """Algorithmic work per launch on the 4096 x 11008 layer: both GEMMs
    2 Cout Cin T flops, the fused permute and the adjoint read (and write)
    the weight-sized matrices once plus one mask bit per weight and P."""
    import lcp_synth
    spec = lcp_synth.DOWN_PROJ_4096x11008
    names = ["layer_init", "sinkhorn_fwd", "permute_mask_unpermute", "error_gemm", "dD_gemm", "block_adjoint"]
    w = bench.kernel_work(spec, names)
    assert w["error_gemm"] == ("flops", 2.0 * 4096 * 11008 * 2048) == w["dD_gemm"]
    kind, nbytes = w["block_adjoint"]
    assert kind == "bytes" and nbytes == 4 * 4096 * 11008 + 4096 * 11008 // 8 + 4 * 172 * 64 * 64
    kind, nbytes = w["permute_mask_unpermute"]
    assert kind == "bytes" and nbytes == 4 * 4096 * 11008 + 4096 * 11008 // 8 + 4 * 172 * 64 * 64
    kind, nbytes = w["layer_init"]
    assert kind == "bytes" and nbytes == 2 * 2048 * 11008 * 2 + 4 * 11008


def test_fused_adjoint_work_and_selection():
    """The bench layer (bf16, B = 64) runs the block adjoint inside the dD
    GEMM: that kernel's work is the GEMM's 2 Cout Cin T flops plus four
    products of 2 Cout Cin B flops (W_b P_b, G_b P_b, and the two sums over
    the rows). The B = 128 layer, fp32 layers and the mask straight-through
    term keep the separate adjoint."""
    import lcp_synth
    spec = lcp_synth.DOWN_PROJ_4096x11008
    assert bench.fused_adjoint(spec) and not bench.fused_adjoint(spec, mask_ste=True)
    assert not bench.fused_adjoint(lcp_synth.CONFIGS[3])           # 13824 x 5120, B = 128
    assert not bench.fused_adjoint(lcp_synth.F32_256x256)
    kind, flops = bench.kernel_work(spec, ["dD_gemm_adjoint"])["dD_gemm_adjoint"]
    assert kind == "flops" and flops == 2.0 * 4096 * 11008 * 2048 + 4 * 2.0 * 4096 * 11008 * 64


def test_source_identity_hashes_the_library_sources():
    ident = bench.source_identity()
    assert len(ident["csrc_sha16"]) == 16
    assert ident["git"] is None or len(ident["git"]) == 12
