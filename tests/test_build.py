"""The build refuses kernels with scratch (register spills): the parser of the
compiler's resource-usage remarks flags them (runs without a GPU)."""
from transformer_attention_rope_amd.build import scratch_kernels


def test_scratch_parser_flags_spilling_kernels():
    t = "\n".join([
        "a.hip:1:1: remark: Function Name: _ZN2nc3fooEv [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 24 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:2:1: remark: Function Name: _ZN2nc3barEv [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:2:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert scratch_kernels(t) == [("_ZN2nc3fooEv", 24)]
    assert scratch_kernels("") == []
