"""The build's scratch guard (CPU): kernels whose pipeline waits count their own
vector loads must not spill, and the guard must find them in the compiler's
resource remarks."""
import pytest

from bit_quantized_grouped_amd import build

NAME = "_ZN5moeq417grouped_q4_kernelILi2ELi32ELi128ELi1ELi2ELi4ELb0ELb1EEEvNS_11GroupedArgsE"
NAME_MT16 = NAME.replace("ELi32ELi128E", "ELi16ELi128E")   # 16-row blocks


def remarks(name, scratch):
    return (f"gemm_q4.hip:1:1: remark: Function Name: {name} [-Rpass-analysis=kernel-resource-usage]\n"
            f"gemm_q4.hip:1:1: remark:     VGPRs: 60 [-Rpass-analysis=kernel-resource-usage]\n"
            f"gemm_q4.hip:1:1: remark:     ScratchSize [bytes/lane]: {scratch} "
            f"[-Rpass-analysis=kernel-resource-usage]\n")


@pytest.mark.parametrize("name", [NAME, NAME_MT16])
def test_counted_wait_kernel_without_scratch_passes(name):
    assert build.check_no_scratch(remarks(name, 0)) == 1


@pytest.mark.parametrize("name", [NAME, NAME_MT16])
def test_counted_wait_kernel_with_scratch_fails(name):
    with pytest.raises(RuntimeError, match="scratch"):
        build.check_no_scratch(remarks(name, 16))


@pytest.mark.parametrize("other", [
    NAME.replace("ELi128E", "ELi64E"),        # 64-K chunks: register-staged x rows
    NAME.replace("ELb0ELb1E", "ELb0ELb0E"),   # separate scale arrays
    NAME.replace("ELb0ELb1E", "ELb1ELb0E"),   # bf16-weight baseline
    "_ZN5moeq418route_fused_kernelILi1EEEvPKfiiiiiNS_10RoutingDevE",
])
def test_other_kernels_are_not_guarded(other):
    assert build.check_no_scratch(remarks(other, 12)) == 0
