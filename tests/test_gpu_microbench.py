"""GPU run of the instruction-throughput microbenchmarks: every benchmark
completes and reports finite positive rates, and the bf16 MFMA issues at the
rate its shape fixes (a 32x32x16 bf16 MFMA occupies a SIMD's matrix core for
32 cycles on gfx950: 1024 FLOP per clock per SIMD)."""

import math

import pytest

pytestmark = pytest.mark.gpu

SMALL_PLAN = tuple((name, wps, max(20, iters // 20))
                   for name, wps, iters in __import__(
                       "head_attention_forward_fmha_amd.microbench",
                       fromlist=["PLAN"]).PLAN)


def test_microbenchmarks_run_and_report_sane_rates():
    import torch
    from head_attention_forward_fmha_amd import microbench
    print("microbench: small plan", flush=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows = microbench.run_all(cus, SMALL_PLAN)
    assert len(rows) == len(SMALL_PLAN)
    for r in rows:
        for k, v in r.items():
            if isinstance(v, float):
                assert math.isfinite(v) and v > 0, (r, k)
    mfma1 = next(r for r in rows if r["bench"] == "mfma_bf16" and r["waves_per_simd"] == 1)
    # 32 cycles by the instruction's shape; allow clock-domain and loop overhead
    assert 31.0 <= mfma1["cycles"] <= 40.0, mfma1
    co = next(r for r in rows if r["bench"] == "mfma_with_valu")
    assert co["valu_cycles_per_iter"] > 0
