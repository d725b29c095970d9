"""The build's scratch-memory check reads the compiler's resource report."""

from linear_attention_recurrent_dl_amd import build

REPORT = """\
x.hpp:1:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]
x.hpp:1:1: remark:     VGPRs: 60 [-Rpass-analysis=kernel-resource-usage]
x.hpp:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hpp:1:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]
x.hpp:1:1: remark:     ScratchSize [bytes/lane]: 144 [-Rpass-analysis=kernel-resource-usage]
x.hpp:1:1: remark: Function Name: kern_c [-Rpass-analysis=kernel-resource-usage]
x.hpp:1:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]
"""


def test_scratch_report_parsing():
    assert build.scratch_kernels(REPORT) == [("kern_b", 144), ("kern_c", 16)]
    assert build.scratch_kernels(REPORT.split("kern_b")[0]) == []
