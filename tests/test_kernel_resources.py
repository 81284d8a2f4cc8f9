"""Kernel resource checks on the CPU (device assembly of the library's own sources):
every kernel runs without a private (scratch) segment.  A kernel whose argument block
the compiler copies to private memory would pay a 1.5 KiB per-lane copy at every launch,
and kernels read their call tables in place in the kernel-argument segment."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_deltanet_recurrent_chunk_amd", "csrc")


@pytest.mark.parametrize("src", ["prefill_kernels.hip", "stream_kernels.hip", "flush_kernel.hip"])
def test_kernels_use_no_private_segment(src, tmp_path):
    out = str(tmp_path / "k.s")
    cmd = ["/opt/rocm/bin/hipcc", "-x", "hip", "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only",
           "-S", "-I", os.path.join(ROOT, "include"), "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-amdgpu-mfma-vgpr-form", os.path.join(CSRC, src), "-o", out]
    if src == "flush_kernel.hip":
        cmd[-2:-2] = ["-mllvm", "-amdgpu-kernarg-preload-count=4"]
    subprocess.run(cmd, check=True, capture_output=True)
    text = open(out).read()
    kernels = re.findall(r"^\t\.amdhsa_kernel (\S+)$", text, re.M)
    sizes = re.findall(r"\.amdhsa_private_segment_fixed_size (\d+)", text)
    assert kernels and len(kernels) == len(sizes)
    bad = [(k, int(n)) for k, n in zip(kernels, sizes) if int(n) > 0]
    assert not bad, bad


def test_prefill_prepass_fits_four_workgroups_per_cu(tmp_path):
    """The pre-pass at d = 128 with bf16 inputs keeps four 4-wave workgroups resident on a
    compute unit: at most 40 KiB of LDS (160 KiB per CU) and 128 VGPRs (512 per SIMD lane
    over four waves)."""
    out = str(tmp_path / "p.s")
    cmd = ["/opt/rocm/bin/hipcc", "-x", "hip", "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only",
           "-S", "-I", os.path.join(ROOT, "include"), "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-amdgpu-mfma-vgpr-form", os.path.join(CSRC, "prefill_kernels.hip"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    text = open(out).read()
    name = "_ZN3gdn16factorize_kernelItLi128EEEvNS_13FactorizeArgsIT_EE"
    lds = re.search(r"\.amdhsa_kernel " + name + r"\n(.*?)\.end_amdhsa_kernel", text, re.S).group(1)
    group = int(re.search(r"\.amdhsa_group_segment_fixed_size (\d+)", lds).group(1))
    vgpr = int(re.search(r"\.set " + name + r"\.num_vgpr, (\d+)", text).group(1))
    assert group <= 40 * 1024, group
    assert vgpr <= 128, vgpr
