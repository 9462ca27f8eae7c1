"""Build check: no kernel uses scratch memory or spills registers.

"10 · R4 — decode split-attention dim-parallel rewrite", sections 2.3 and 6:
an accumulator sized at run time went to local memory and cost most of the
old kernel's time; the accumulators here are sized at compile time and must
stay in registers. The compiler's per-kernel resource report (written by
decode_attention_gqa_amd/build.py) is checked for every instantiation.
"""
import os
import re

import pytest

from decode_attention_gqa_amd import build


def _report():
    if not os.path.exists(build.RESOURCE_REPORT) or not os.path.exists(build.LIB):
        build.build()
    with open(build.RESOURCE_REPORT) as f:
        return f.read()


def _kernels(text):
    """{mangled name: {field: value}} from the resource-usage remarks."""
    out, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^]]+\])?: (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return out


def test_every_kernel_without_scratch_or_spills():
    ks = _kernels(_report())
    partial = [k for k in ks if "partial_" in k]
    # template arguments <HD, G, PER_HEAD, R, FOLD>: the per-head form has
    # PER_HEAD = true, R = 1; the decode-step form FOLD = true
    per_head = [k for k in partial if re.search(r"ELb1ELi1ELb0EE", k)]
    rows = [k for k in partial if re.search(r"ELb0ELi[248]ELb0EE", k)]
    fold = [k for k in partial if re.search(r"ELb0ELi1ELb1EE", k)]
    # 6 head dims x 8 group sizes, the 3 per-query-head forms (hd 64/128/256),
    # 7 one-block (group, rows) forms for several query rows x 3 head dims
    # and 7 two-block forms ((2, 8), (3, 4), (4, 4), (5..8, 2)) x hd 64/128,
    # the decode-step form for 8 group sizes x 3 head dims, plus combine,
    # append and probe kernels
    assert (len(partial) == 110 and len(per_head) == 3 and len(rows) == 35
            and len(fold) == 24), (len(partial), len(per_head), len(rows),
                                   len(fold))
    assert any("combine_kernel" in k for k in ks)
    for name, f in ks.items():
        assert f.get("ScratchSize", 0) == 0, (name, f)
        assert f.get("VGPRs Spill", 0) == 0, (name, f)
        assert f.get("SGPRs Spill", 0) == 0, (name, f)


@pytest.mark.parametrize("hd,g,occ", [(128, 7, 4), (64, 8, 7), (256, 8, 2)])
def test_matrix_core_kernel_occupancy(hd, g, occ):
    ks = _kernels(_report())
    name = [k for k in ks if f"partial_mfma_kernelILi{hd}ELi{g}ELb0ELi1ELb0EE" in k]
    assert name, (hd, g)
    f = ks[name[0]]
    assert f.get("Occupancy", 0) >= occ, f


LDS_PER_CU = 160 * 1024


def _wg_per_cu(name, f):
    """Resident workgroups per compute unit from the compiler report: waves
    per SIMD x 4 SIMDs / waves per workgroup (8 for the head_dim-256
    matrix-core kernel, else 4), capped by the LDS of a compute unit."""
    waves = 8 if re.search(r"partial_mfma_kernelILi256E", name) else 4
    by_regs = f["Occupancy"] * 4 // waves
    lds = f.get("LDS Size [bytes/block]", f.get("LDS Size", 0))
    by_lds = LDS_PER_CU // lds if lds else by_regs
    return min(by_regs, by_lds)


def test_workgroups_per_cu_matches_compiler_report(splitkv_lib_path):
    """The split heuristic sizes one round of workgroups from the library's
    occupancy table; it must equal what the compiler reports for each
    (head_dim, group) instantiation."""
    import decode_attention_gqa_amd as skv
    ks = _kernels(_report())
    seen = 0
    for name, f in ks.items():
        m = re.search(r"partial_(?:mfma|valu)_kernelILi(\d+)ELi(\d+)E", name)
        if not m or re.search(r"ELb1ELi1ELb0EE|ELb0ELi[248]ELb0EE|ELb1EE", name):
            continue   # the per-head, several-row and decode-step forms aside
        hd, g = int(m.group(1)), int(m.group(2))
        assert skv.workgroups_per_cu(hd, g) == _wg_per_cu(name, f), (hd, g, f)
        seen += 1
    assert seen == 48
    # the one-block several-row forms fit as many workgroups per CU as the
    # one-row form; the two-block forms (twice the accumulators) keep one
    # round of the heuristic's workgroups resident (256 / hd per CU)
    for name, f in ks.items():
        m = re.search(r"partial_mfma_kernelILi(\d+)ELi(\d+)ELb0ELi([248])ELb0EE", name)
        if m:
            hd, g, r = int(m.group(1)), int(m.group(2)), int(m.group(3))
            if g * r <= 8:
                assert skv.workgroups_per_cu(hd, g) == _wg_per_cu(name, f), \
                    (name, f)
            else:
                assert _wg_per_cu(name, f) >= 256 // hd, (name, f)
    # the decode-step form keeps one round of the heuristic's workgroups
    # resident (at most 256 / hd per compute unit for one sequence)
    for name, f in ks.items():
        m = re.search(r"partial_mfma_kernelILi(\d+)ELi(\d+)ELb0ELi1ELb1EE", name)
        if m:
            hd = int(m.group(1))
            assert _wg_per_cu(name, f) >= 256 // hd, (name, f)
    assert skv.workgroups_per_cu(96, 4) == 0
    assert skv.workgroups_per_cu(128, 9) == 0
