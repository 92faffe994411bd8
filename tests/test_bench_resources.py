"""CPU tests of the resource entry the bench line carries: for every workload
the bench times, the compiler's report (written by the build next to the
library) holds the timed kernel, with no scratch and no spills."""

import dataclasses
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REPORT = os.path.join(ROOT, "head_attention_forward_fmha_amd", "libfmha.resource-usage.txt")

pytestmark = pytest.mark.skipif(not os.path.exists(REPORT), reason="library not built")


def _bench():
    spec = importlib.util.spec_from_file_location("fmha_bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _clean(entry):
    assert entry is not None
    assert entry["scratch_bytes_per_lane"] == 0
    assert entry["vgpr_spill"] == 0 and entry["sgpr_spill"] == 0
    assert 0 < entry["vgprs"] <= 512 and entry["occupancy_waves_per_simd"] >= 1
    assert entry["lds_bytes_per_block"] <= 160 * 1024


@pytest.mark.parametrize("variant", ["pingpong", "four_wave"])
@pytest.mark.parametrize("name", ["c2_dense_2225", "c3_varlen_causal_8k", "c4_varlen_causal_32k",
                                  "c5_causal_fp8pv_32k", "x_causal_fp4pv_32k"])
def test_forward_kernel_of_each_workload_is_in_the_report(name, variant):
    from synthetic import EXTRA_WORKLOADS, WORKLOADS
    w = {**WORKLOADS, **EXTRA_WORKLOADS}[name]
    bench = _bench()
    for split in (False, True):
        if split and (w.fp4_pv or w.fp8_pv):
            continue  # split-KV is built for bf16 P.V only
        entry = bench.timed_kernel_resources(w, variant, split)
        _clean(entry)
        assert entry["symbol"].startswith("_ZN4fmha")


def test_c4_pingpong_entry_matches_its_design():
    from synthetic import WORKLOADS
    e = _bench().timed_kernel_resources(WORKLOADS["c4_varlen_causal_32k"], "pingpong")
    _clean(e)
    # 8 waves of 256 VGPRs at most: two waves per SIMD; three K/V stages of
    # 2 x 64 x 128 bf16 in LDS, and the epilogue's private 4 KB O block per wave
    assert e["vgprs"] <= 256 and e["occupancy_waves_per_simd"] == 2
    assert e["lds_bytes_per_block"] == 3 * 2 * 64 * 128 * 2 + 8 * 4096


@pytest.mark.parametrize("causal", [True, False])
def test_backward_kernels_are_in_the_report(causal):
    from synthetic import WORKLOADS
    w = WORKLOADS["c4_varlen_causal_32k"]
    w = dataclasses.replace(w, causal=causal)
    res = _bench().bwd_kernel_resources(w)
    assert sorted(res) == ["dkdv", "dq"]
    for entry in res.values():
        _clean(entry)


def test_missing_report_gives_none(tmp_path):
    from head_attention_forward_fmha_amd import build
    assert build.kernel_resources("_ZN4fmha_x", str(tmp_path / "none.txt")) is None
    p = tmp_path / "r.txt"
    p.write_text("a.hip:1:1: remark: Function Name: k [-Rpass-analysis=kernel-resource-usage]\n"
                 "a.hip:1:1: remark:     VGPRs: 12 [-Rpass-analysis=kernel-resource-usage]\n")
    assert build.kernel_resources("other", str(p)) is None
    assert build.kernel_resources("k", str(p))["vgprs"] == 12
