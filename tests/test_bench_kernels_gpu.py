"""The kernel list bench.py prices (its roofline, traffic and profile
summaries) against the kernels the library actually dispatches.

bench.py mirrors the library's host-side choices (decode pair or tiled GEMM,
which shrink, whether the d_in split needs k_vfinal, device segmentation,
whether the adapter term is added as a dense tile) in
Python. With MLORA_LOG=1 the library prints the path, the d_in split and the
shrink it took; the two must agree on every bench workload, LoRA-on.
"""
import re

import pytest

from gpu_util import DeviceCase, log
from mlora_inputs import make_case

pytestmark = pytest.mark.gpu

WORKLOADS = [("tiny_f32", "q"), ("decode_bf16", "q"), ("verify_bf16", "q"), ("hetero_bf16", "q"),
             ("prefill_bf16", "q"), ("prefill_bf16", "k")]


def _logged(dc, capfd):
    capfd.readouterr()
    dc.run(1)
    err = capfd.readouterr().err
    m = re.search(r"mlora: path=(\S+) T=\d+ .* ks=(\d+) shrink=(\S+) ", err)
    assert m, err
    return m.group(1), int(m.group(2)), m.group(3)


@pytest.mark.parametrize("name,proj", WORKLOADS)
def test_bench_kernel_list_matches_dispatch(name, proj, monkeypatch, capfd):
    import bench
    log(f"[bench kernels] {name} {proj}")
    case = make_case(name, proj)
    dc = DeviceCase(case)
    monkeypatch.setenv("MLORA_LOG", "1")
    path, ks, shrink = _logged(dc, capfd)
    kernels = bench.layer_kernels(case)
    expect_path = {"bf16": "gemm", "f32": "f32"}[case.dtype]
    if kernels == ["k_stream_bf16", "k_finish_bf16"]:
        expect_path = "decode"
    elif "k_expand_delta" in kernels:
        expect_path = "gemm-dense-expand"
    assert path == expect_path, (path, kernels)
    if path in ("gemm", "gemm-dense-expand"):
        assert ks == bench.shrink_split(case), (ks, bench.shrink_split(case))
        # (the dense term's expand folds the shrink's chunks itself)
        assert ("k_vfinal" in kernels) == (ks > 1 and path != "gemm-dense-expand")
        assert ("k_shrink_short" in kernels) == (shrink == "short"), (shrink, kernels)
        assert ("k_shrink2" in kernels) == (shrink == "mfma"), (shrink, kernels)
        assert ("k_build_segments" in kernels) == (not case.sorted_input)
    elif path == "f32":
        assert kernels == ["k_shrink_f32", "k_gemm_f32"]
    monkeypatch.setenv("MLORA_FORCE_SHRINK", "mfma")
    if path == "gemm":   # the switch that keeps the MFMA shrink is mirrored too
        path2, _, shrink2 = _logged(dc, capfd)
        assert shrink2 == "mfma" and "k_shrink2" in bench.layer_kernels(case)
