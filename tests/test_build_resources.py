"""Register and scratch budgets of the built kernels (CPU; reads the compiler's resource report).

`python -m int6_weight_export_amd.build` records, per kernel, the VGPRs, scratch bytes per lane,
occupancy and spills that the compiler reports (-Rpass-analysis=kernel-resource-usage) in
int6_weight_export_amd/_build/resources.json.  A kernel that spills into scratch or loses
occupancy streams far slower: an out-of-line call left in a row path once took the
percentile-select export from 48 to 311 us.  These budgets catch that at build time.
"""
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RES = os.path.join(ROOT, "int6_weight_export_amd", "_build", "resources.json")

pytestmark = pytest.mark.skipif(not os.path.exists(RES), reason="library not built here (no resource report)")


def _load():
    with open(RES) as f:
        return json.load(f)


def _table(res, mode, feats):
    pat = re.compile(rf"pgq_table_kernelILi{mode}ELj{feats}E")
    hits = [v for k, v in res.items() if pat.search(k)]
    assert len(hits) == 1, (mode, feats, len(hits))
    return hits[0]


def test_grouped_kernels_use_no_scratch():
    res = _load()
    # the all-features candidate pass (mixed or unaligned per-tensor calls only) is the exception
    bad = {k: v for k, v in res.items() if "pgq_table_kernel" in k and v.get("scratch", 0) > 0
           and "ILi9ELj163E" not in k}
    assert not bad, bad
    assert all(v.get("vgpr_spill", 0) == 0 for k, v in res.items() if "ILi9ELj163E" not in k), \
        {k: v for k, v in res.items() if v.get("vgpr_spill", 0)}


def test_other_kernels_stay_within_small_scratch():
    res = _load()
    assert all(v.get("scratch", 0) <= 32 for v in res.values()), {k: v for k, v in res.items() if v.get("scratch", 0) > 32}


@pytest.mark.parametrize("mode,feats,max_vgprs,min_occ", [
    (0, 5, 72, 7),      # fp32 export with passthrough (the headline kernel)
    (0, 6, 80, 6),      # bf16 export
    (0, 21, 128, 4),    # fp32 export with the per-row percentile select
    (7, 5, 72, 7),      # export with 6-bit codes
    (1, 5, 96, 5),      # SQWA
    (2, 2, 128, 4),     # STE forward + backward, bf16
    (4, 1, 64, 8),      # EMA, fp32
    (9, 1, 96, 5),      # candidate pass, fp32
])
def test_streaming_kernel_budgets(mode, feats, max_vgprs, min_occ):
    v = _table(_load(), mode, feats)
    assert v["vgprs"] <= max_vgprs and v["occupancy"] >= min_occ, v


def test_gemm_fits_without_scratch():
    res = _load()
    g = [v for k, v in res.items() if re.search(r"pgq_qgemm_kernel", k)]     # fp32 and bf16 Y
    assert len(g) == 2 and all(v["scratch"] == 0 and v["occupancy"] >= 2 for v in g), g


def test_tensor_pick_is_one_inlined_kernel():
    """The whole-tensor pick keeps its candidate ranking inline: compiled as an out-of-line call
    it needed 12 bytes of scratch per lane and 102 VGPRs, and the pick took 12.0 instead of
    10.9 us."""
    res = _load()
    p = [v for k, v in res.items() if "pgq_tensor_pick_kernel" in k]
    assert len(p) == 1 and p[0]["scratch"] == 0 and p[0]["vgprs"] <= 80, p
