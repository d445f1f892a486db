"""Compiled matrix-core code reads no result before its wait states (CPU: device assembly only).

The 16x16x128 dense 8-bit instruction takes twice the cycles of the 8-bit sparse one.  Where both
wrote one accumulator on the two arms of a tile-type branch, the compiler read it after the join
with the shorter instruction's wait states, and the products came out wrong.  This test compiles
the product kernels with the library's own flags and walks every path of the result.
"""
from __future__ import annotations

import os
import tempfile

import pytest

from tile_gemm_amd import build as hb

from isa_waitstates import PROBE_OPS, required_waits, device_asm, violations

SOURCES = ["gemm_prefill.hip", "gemm_decode.hip"]


def _hipcc():
    try:
        return hb.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")


def _flags():
    return [f for f in hb.COMMON if f != "-fPIC"] + hb.VGPR_FORM


@pytest.fixture(scope="module")
def need():
    w = required_waits(_flags(), _hipcc())
    assert set(w) == set(PROBE_OPS), f"probe did not show every instruction: {sorted(w)}"
    return w


def test_probe_wait_states_are_plausible(need):
    # a result is never readable on the next cycle, and the dense 8-bit 16x16x128 form
    # (twice the cycles of the 8-bit sparse form) needs more than it
    assert all(v >= 4 for v in need.values()), need
    assert need["v_mfma_scale_f32_16x16x128_f8f6f4"] > need["v_smfmac_f32_16x16x128_fp8_fp8"], need


def test_checker_flags_a_short_wait(need):
    w = need["v_mfma_scale_f32_16x16x128_f8f6f4"]
    short = f"""k:
\tv_mfma_scale_f32_16x16x128_f8f6f4 v[8:11], v[0:7], v[12:19], v[8:11], v1, v1
\ts_cbranch_scc1 .L1
\ts_nop {w - 4}
.L1:
\tv_mov_b64_e32 v[20:21], v[8:9]
\ts_endpgm
"""
    assert len(violations(short, need)) == 1
    enough = short.replace(f"s_nop {w - 4}", f"s_nop {w - 2}").replace("s_cbranch_scc1 .L1", "s_nop 0")
    assert violations(enough, need) == []
    chained = short.replace("v_mov_b64_e32 v[20:21], v[8:9]",
                            "v_mfma_scale_f32_16x16x128_f8f6f4 v[8:11], v[0:7], v[12:19], v[8:11], v1, v1")
    assert violations(chained, need) == []


@pytest.mark.parametrize("src", SOURCES)
def test_product_kernels_respect_wait_states(need, src):
    with tempfile.TemporaryDirectory() as d:
        text = device_asm(os.path.join(hb.CSRC, src), os.path.join(d, "k.s"), _flags(), _hipcc())
    bad = violations(text, need)
    assert not bad, f"{len(bad)} early reads, first: {bad[:3]}"
