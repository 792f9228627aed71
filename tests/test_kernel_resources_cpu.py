"""The hot kernels' register budgets, from the compiler's resource report that the build
writes (_build/kernel_resources.json): every forward and gradient matrix-core kernel keeps
two waves per SIMD (two workgroups of four waves per CU, as the work plans assume), the
forward kernels spill nothing except the d = dv = 128 kernel with a bias, and no kernel
spills more than the few registers these variants are known to. A regression here (for
example the compiler sinking the 16-bit conversions again, which made that kernel spill
91 registers and run 2.2x slower) fails before any GPU run. Skipped when the library has
not been built in this tree.
"""

import json
import os
import re

import pytest

REPORT = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "_build", "kernel_resources.json")

pytestmark = pytest.mark.skipif(not os.path.exists(REPORT), reason="no build report (run __graft_entry__.build())")


def _kernels(kind):
    rep = json.load(open(REPORT))
    pat = re.compile(kind + r"I(DF16b|DF16_)Li(\d+)ELi(\d+)ELb([01])E")
    out = {}
    for name, res in rep.items():
        m = pat.search(name)
        if m:
            out[(m.group(1), int(m.group(2)), int(m.group(3)), m.group(4) == "1")] = res
    return out


# most spilled registers allowed per variant (d, dv, bias); absent: none
FWD_SPILL_MAX = {(128, 128, True): 16}
BWD_SPILL_MAX = {(128, 128, False): 16, (128, 128, True): 40}


@pytest.mark.parametrize("kind,limits", [("8fwd_mfma", FWD_SPILL_MAX), ("8bwd_mfma", BWD_SPILL_MAX)])
def test_matrix_core_kernels_keep_two_waves_and_their_registers(kind, limits):
    ks = _kernels(kind)
    assert len(ks) == 16, f"expected 16 {kind} variants in the report, found {len(ks)}"
    for (et, d, dv, bias), res in ks.items():
        where = f"{kind}<{et}, {d}, {dv}, bias={bias}>"
        assert res["Occupancy [waves/SIMD]"] >= 2, where
        assert res["VGPRs Spill"] <= limits.get((d, dv, bias), 0), (where, res["VGPRs Spill"])
        assert res["SGPRs Spill"] == 0, where
