"""The hardware costs the kernel design rests on, measured on the GPU (tests/hw/hw_costs.hip,
built by __graft_entry__.build()): the relations below are what the design uses, with
wide margins (the printed numbers are the measurement).

* the FP6 scaled MFMA runs at about half the cycles of the FP8 one (why INT4 codes go
  through FP6 E2M3 operands);
* VALU work next to an MFMA in the same wave mostly serializes with it (why the INT4
  rescale's v_fmac count bounds kernel 2);
* the two-block v_mfma_f32_32x32x4_2b_f16 has the documented operand / result layout;
* LDS-destination buffer loads and ds_read_b128 deliver far more than kernel 2 moves (so
  the loads' bandwidth is not its bound), and 16-byte loads staged through registers
  reach the same L2 -> CU rate as the LDS-destination loads (no faster path to LDS);
* an FP6 MFMA stream in one wave and a v_fmac stream in another wave of the same SIMD
  only partly overlap: each MFMA takes VALU issue cycles from the other wave (why the
  INT4 rescale's VALU work and its MFMAs add up rather than overlap).
"""
import json
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hw", "hw_costs")


def test_hardware_costs():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: run __graft_entry__.build() first")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=180)
    assert r.returncode == 0, r.stderr[-2000:]
    rows = [json.loads(l) for l in r.stdout.splitlines() if l.startswith("{")]
    for row in rows:
        print(row, flush=True)
    cyc = {(x["what"], x.get("waves_per_simd")): x.get("cycles") for x in rows}
    bw = {x["what"]: x["bytes_per_cycle_cu"] for x in rows if "bytes_per_cycle_cu" in x}
    fp6, fp8 = cyc[("mfma_fp6_32x32x64", 1)], cyc[("mfma_fp8_32x32x64", 1)]
    assert fp8 > 1.5 * fp6
    # 16 independent v_fmac after each MFMA of one wave: most of their time adds
    alone, both = cyc[("same_wave_fp6_mfma_plus_0_fmac", 1)], cyc[("same_wave_fp6_mfma_plus_16_fmac", 1)]
    fmac = cyc[("valu_fmac", 1)]
    assert both > alone + 0.5 * 16 * fmac
    assert [x for x in rows if x["what"] == "mfma_32x32x4_2b_f16_layout"][0]["ok"] == 1
    assert bw["lds_dma_l2_8_in_flight_2_blocks"] > 20
    assert bw["ds_read_b128_8_waves_per_cu"] > 64
    reg, lds_dma = bw["reg_load_ds_write_l2_8_in_flight_2_blocks"], bw["lds_dma_l2_8_in_flight_2_blocks"]
    assert 0.5 < reg / lds_dma < 2.0
    cr = {x["what"]: x["cycles_per_iter"] for x in rows if x["what"].startswith("cross_")}
    m, v, both = cr["cross_mfma_only"], cr["cross_valu_only"], cr["cross_mfma_and_valu_waves"]
    assert max(m, v) * 1.15 < both < m + v
    # the double-rate VALU class (fp32 fma / mul / add, bitwise and) against the single-rate
    # class (mixed-precision fma, shifts, conversions) that the kernels' inner loops avoid
    fast = [cyc[("valu_" + n, 8)] for n in ("v_fmac_f32", "v_mul_f32", "v_and_b32", "v_add_f32")]
    slow = [cyc[("valu_" + n, 8)] for n in ("v_fma_mix_f32", "v_lshlrev_b32", "v_cvt_f32_f16")]
    assert max(fast) * 1.2 < min(slow)
