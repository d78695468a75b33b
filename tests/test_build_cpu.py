"""The build refuses kernels that spill registers to scratch memory: a
spilled hot loop runs at a fraction of its speed and nothing else reports it.
The check reads the compiler's per-kernel resource report; these cases pin
the reader on report text of the form the compiler prints."""
import pytest

from bit_weight_only_amd.build import scratch_kernels

REPORT = """\
k.hip:10:1: remark: Function Name: _Z3fooPf [-Rpass-analysis=kernel-resource-usage]
k.hip:10:1: remark:     VGPRs: 128 [-Rpass-analysis=kernel-resource-usage]
k.hip:10:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
k.hip:20:1: remark: Function Name: _Z3barPf [-Rpass-analysis=kernel-resource-usage]
k.hip:20:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
k.hip:20:1: remark:     ScratchSize [bytes/lane]: 560 [-Rpass-analysis=kernel-resource-usage]
k.hip:20:1: remark:     VGPRs Spill: 227 [-Rpass-analysis=kernel-resource-usage]
k.hip:30:1: remark: Function Name: _Z3bazPf [-Rpass-analysis=kernel-resource-usage]
k.hip:30:1: remark:     ScratchSize [bytes/lane]: 12 [-Rpass-analysis=kernel-resource-usage]
"""


def test_scratch_kernels_names_only_the_spilling_kernels():
    assert scratch_kernels(REPORT) == [("_Z3barPf", 560), ("_Z3bazPf", 12)]


def test_scratch_kernels_empty_report():
    assert scratch_kernels("") == []
    assert scratch_kernels(REPORT.split("k.hip:20")[0]) == []


@pytest.mark.parametrize("line", ["warning: foo", "remark: VGPRs: 3"])
def test_scratch_kernels_ignores_other_lines(line):
    assert scratch_kernels(line) == []
