"""Host logic of bench.py (CPU only): dispatch names from a kernel trace map to
the workloads whose rates and traffic the bench reports, and every workload
belongs to the kernel family whose sources its traffic figure is keyed to.

The names are the demangled forms rocprofv3 records for the shipped launch
shapes; the grid sizes follow from the launch code for the bench's sizes.
"""
from __future__ import annotations

import pytest

import bench

NS = "void q4k::(anonymous namespace)::"

# (kernel with template arguments, total work-items of the launch, LDS bytes, hint) -> workload
CASES = [
    ("k_gemv_decode<8, 1, false, 4>", 4096 // 8 * 512, 17408, "", "gemv_4096x4096"),
    ("k_gemv_decode<8, 4, false, 4>", 4096 // 8 * 512, 69632, "mlp", "swiglu_mlp_down_4096x14336"),
    ("k_gemv_decode<8, 1, true, 4>", 14336 // 4 * 512, 17920, "mlp",
     "swiglu_mlp_gateup_14336x4096"),
    ("k_gemv_decode<8, 1, false, 4>", 14336 // 8 * 512, 17408, "", "sweep_gemv_14336x4096_m1"),
    ("k_gemv_decode<8, 1, false, 5>", 4096 // 8 * 512, 17408, "", "q5k_gemv_4096x4096"),
    ("k_gemv_q4k<2, 2, false, 4, 4>", 196608, 0, "", "sweep_gemv_14336x4096_batched"),
    ("k_gemv_q4k<1, 1, true, 8, 4>", 4096, 0, "", "swiglu_mlp_gateup_other"),
    ("k_gemm_q4k_kslice<2, 2, 4>", 131072, 163840, "", "gemm_512x4096x4096"),
    ("k_gemm_q4k_kslice<2, 2, 5>", 131072, 157696, "", "q5k_gemm_512x4096x4096"),
    ("k_gemm_q4k_kslice<1, 2, 4>", 224 * 256, 81920, "", "sweep_gemm_14336x4096"),
    ("k_gemm_q4k_stream<1, 8>", 448 * 256, 57344, "", "sweep_gemm_14336x4096"),
    ("k_gemm_q4k_stream<2, 32>", 224 * 256, 155648, "", "sweep_gemm_14336x4096"),
    ("k_gemm_q4k_128x256", 57344, 155648, "", "gemm_512x14336x4096"),
    ("k_gemm_planes_lds<6>", 32 * 4 * 2 * 512, 151552, "", "q6k_gemm_512x4096x4096"),
    ("k_gemm_planes_lds<3>", 32 * 4 * 2 * 512, 135168, "", "q3k_gemm_512x4096x4096"),
    ("k_gemm_planes<6, 4, 1, 1, 4>", 128 * 2 * 256, 36864, "", "q6k_gemm_512x4096x4096"),
    ("k_gemv_planes<6, 8, 2, 1>", 4096 // 16 * 512, 16384, "", "q6k_gemv_4096x4096"),
    ("k_gemv_planes_lds<6, 4, 1, 1>", 4096 // 4 * 256, 32768, "", "q6k_gemv_4096x4096"),
    ("k_gemv_planes_lds<3, 4, 1, 1>", 4096 // 4 * 256, 24576, "", "q3k_gemv_4096x4096"),
    ("k_gemv_planes_lds<3, 8, 2, 4>", 4096 // 16 * 512, 90112, "", "planes_other"),
    ("k_gemv_split<1, 2, 4>", 0, 0, "", "sweep_gemv_14336x4096_split"),
    ("k_gemv_layers", 256 * 1024, 0, "", "gemv_layers_8x4096x4096"),
    ("k_w8a8_gemm<1, 3, 3, 1>", 16 * 16 * 256, 98304, "", "w8a8_linear_1024x3072x3072"),
    ("k_w8a8_gemm<2, 3, 2, 1>", 16 * 64 * 256, 81920, "", "w8a8_linear_8192x3072x3072"),
    ("k_w8a8_gemm<2, 2, 2, 1>", 24 * 64 * 256, 65536, "", "w8a8_other"),
    ("k_w8a8_quantize_rows<8>", 1024 * 64, 0, "", "w8a8_quantize_1024x3072"),
    ("k_zero_planes", 524544, 0, "", "split_k_zero_fill"),
    ("k_zero_f32", 524544, 0, "", "split_k_zero_fill"),
]


@pytest.mark.parametrize("kernel,threads,lds,hint,workload", CASES)
def test_dispatch_names_map_to_bench_workloads(kernel, threads, lds, hint, workload):
    name = NS + kernel + "(unsigned char const*, float*, int, int, int)"
    assert bench.dispatch_workload(name, threads, lds, hint) == workload


def test_template_arguments_parse():
    assert bench._template_args(NS + "k_gemm_q4k_kslice<2, 1, 5>(int)", "k_gemm_q4k_kslice") == \
        ("2", "1", "5")
    assert bench._template_args(NS + "k_gemm_q4k_kslice<2, 1, 5>(int)", "k_gemm_q4k") is None


@pytest.mark.parametrize("workload,family", [
    ("gemv_4096x4096", "gemv"), ("swiglu_mlp_down_4096x14336", "gemv"),
    ("sweep_gemv_14336x4096_split", "gemv"), ("gemv_layers_8x4096x4096", "gemv"), ("gemm_512x4096x4096", "gemm"),
    ("q5k_gemm_512x4096x4096", "gemm"), ("sweep_gemm_14336x4096", "gemm"),
    ("q6k_gemm_512x4096x4096", "planes"), ("q3k_gemv_4096x4096", "planes"),
    ("dequant_bf16_4096x4096", "dequant"), ("w8a8_linear_1024x3072x3072", "w8a8"),
])
def test_workloads_key_their_traffic_to_their_sources(workload, family):
    assert bench._family(workload) == family
    assert family in bench.KERNEL_SOURCES
